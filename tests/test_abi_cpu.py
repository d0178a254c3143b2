"""C-ABI checks that need no GPU: the library loads, exports every function
include/tokengate.h declares, and rejects invalid arguments on the host
before any HIP call (NULL device pointers are fine: nothing is launched)."""

import ctypes
import os
import re

import pytest

import learned_token_pruning_layer_amd as tg
from learned_token_pruning_layer_amd._lib import TgGather, seq_array
from synthetic import Prompt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return tg.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 22, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(tg.EXPORTED)


def test_status_strings(lib):
    for code in range(5):
        assert lib.tg_status_string(code)


def test_kept_rows_and_validation(lib):
    ps = [Prompt(0, 16384, 0, 16000, 2000)]
    assert tg.tg_kept_rows(ps) == 2384
    ragged = [Prompt(0, 100, 10, 90, 5), Prompt(100, 50, 0, 50, 50), Prompt(150, 0, 0, 0, 0)]
    assert tg.tg_kept_rows(ragged) == (5 + 20) + 50 + 0
    bad = [
        [Prompt(0, 10, 0, 8, 9)],                          # k_doc > n_doc
        [Prompt(0, 10, 0, 8, -1)],                         # k_doc < 0
        [Prompt(0, 10, 3, 2, 0)],                          # doc_begin > doc_end
        [Prompt(0, 10, 0, 11, 0)],                         # doc_end > len
        [Prompt(0, -1, 0, 0, 0)],                          # negative length
        [Prompt(5, 10, 0, 5, 1), Prompt(8, 10, 0, 5, 1)],  # overlapping prompts
    ]
    for b in bad:
        assert lib.tg_kept_rows(seq_array(b), len(b)) == -1
        assert lib.tg_last_error()
    many = [Prompt(i, 1, 0, 1, 1) for i in range(tg.TG_MAX_SEQS + 1)]
    assert lib.tg_kept_rows(seq_array(many), len(many)) == -1


def test_select_rejects_before_launch(lib):
    bad = [Prompt(0, 10, 0, 8, 9)]
    st = lib.tg_select_topk(None, seq_array(bad), 1, None, None, 0, None)
    assert st == INVALID and b"k_doc" in lib.tg_last_error()
    ok = [Prompt(0, 10, 0, 8, 3)]
    assert lib.tg_select_topk(None, seq_array(ok), 1, None, None, 0, None) == INVALID  # NULL scores
    assert lib.tg_select_workspace_bytes(seq_array(ok), 1) == 0
    # Prompts above 32768 rows take the multi-workgroup select, which needs a
    # workspace: per long prompt 3 histograms of 2048 words and 3 x 4 state
    # words, plus per 16384-row chunk of the prompt 4 count words and a
    # candidate list of 16384 words.
    long = [Prompt(0, 100, 0, 90, 5), Prompt(100, 40000, 0, 39000, 7), Prompt(40100, 131072, 0, 130048, 8128)]
    need = lib.tg_select_workspace_bytes(seq_array(long), 3)
    assert need == 4 * (2 * (3 * 2048 + 12) + (3 + 8) * (4 + 16384))
    # Missing or short workspace is refused before anything is enqueued (the
    # pointers below are never dereferenced).
    fake = ctypes.c_void_p(4096)
    assert lib.tg_select_topk(fake, seq_array(long), 3, fake, None, 0, None) == WORKSPACE
    assert b"needed" in lib.tg_last_error()
    assert lib.tg_select_topk(fake, seq_array(long), 3, fake, fake, need - 1, None) == WORKSPACE


def test_decode_table_and_rejects_before_launch(lib):
    from learned_token_pruning_layer_amd._lib import kv_seq_array
    # Workspace: one partial (max, sum, O[D]) per query slot for each wave;
    # a wave covers kpw keys of one (sequence, KV head). 16 heads over 8 KV
    # heads with one new token: 2 query slots. kpw is the smallest power of
    # two >= 32 (bf16, head_dim 128: 4 lane groups x 8 keys) giving at most
    # ~4096 waves and at most 256 splits per sequence: 9152 rows -> 64, so
    # 143 + 47 splits for 9152 + 3000 rows.
    segs = [(0, 9152, 1), (9152, 3000, 1), (12152, 10, 0)]
    need = lib.tg_decode_workspace_bytes(kv_seq_array(segs), 3, 16, 8, 128)
    assert need == (143 + 47) * 8 * 2 * (128 + 2) * 4
    assert lib.tg_decode_workspace_bytes(kv_seq_array([(0, 5, 0)]), 1, 16, 8, 128) == 0
    fake = ctypes.c_void_p(4096)
    args = (fake, fake, fake, fake, fake, kv_seq_array(segs), 3, 16, 8, 128, fake, 1.0, fake, None)
    assert lib.tg_decode_attention(1, *args, None, 0, None) == WORKSPACE
    assert lib.tg_decode_attention(1, *args, fake, need - 4, None) == WORKSPACE
    # (hq/hkv) * n_new above 8, n_new beyond the cache, bad head_dim, bad tau
    assert lib.tg_decode_attention(1, fake, fake, fake, fake, fake, kv_seq_array([(0, 9, 5)]), 1, 16, 8, 128,
                                   fake, 1.0, fake, None, fake, 1 << 20, None) == UNSUPPORTED
    assert lib.tg_decode_attention(1, fake, fake, fake, fake, fake, kv_seq_array([(0, 3, 4)]), 1, 16, 8, 128,
                                   fake, 1.0, fake, None, fake, 1 << 20, None) == INVALID
    assert lib.tg_decode_attention(1, fake, fake, fake, fake, fake, kv_seq_array([(0, 3, 1)]), 1, 16, 8, 96,
                                   fake, 1.0, fake, None, fake, 1 << 20, None) == UNSUPPORTED
    assert lib.tg_decode_attention(1, fake, fake, fake, fake, fake, kv_seq_array([(0, 3, 1)]), 1, 16, 8, 128,
                                   fake, 0.0, fake, None, fake, 1 << 20, None) == INVALID
    # nothing to decode: OK without any pointer
    assert lib.tg_decode_attention(1, None, None, None, None, None, kv_seq_array([(0, 3, 0)]), 1, 16, 8, 128,
                                   None, 1.0, None, None, None, 0, None) == 0


def test_backward_workspace_and_rejects_before_launch(lib):
    # Workspace (fp32 words): the softmax row term [hq][M]; for each of the two
    # halves a (block, head) is split into when the items are few (here: 5 blocks
    # x 16 heads): dK and dV partials [hq][M][D], bias partials and
    # sum_i dS (q . k) partials [hq][M] each, and dQ partials [M][hq][D].
    prompts = [Prompt(0, 100, 0, 90, 40), Prompt(100, 70, 0, 0, 0)]  # 50 and 70 kept rows
    m, hq, hkv, d = 120, 16, 8, 128
    need = lib.tg_attention_backward_workspace_bytes(seq_array(prompts), 2, hq, hkv, d)
    assert need == 4 * (hq * m * (1 + 2 * (3 * d + 2)))
    # Without the split (enough blocks): no dQ partials, one set of the others.
    big = [Prompt(0, 5000, 0, 0, 0)]
    mb = 5000
    need_big = lib.tg_attention_backward_workspace_bytes(seq_array(big), 1, hq, hkv, d)
    assert need_big == 4 * (hq * mb * (1 + 2 * d + 2))
    fake = ctypes.c_void_p(4096)
    args = [fake, fake, fake, fake, fake, seq_array(prompts), 2, hq, 8, d, fake, 1.2, fake, fake, fake,
            fake, fake, fake, fake, fake, fake]
    assert lib.tg_gated_attention_backward(0, *args, fake, need, None) == UNSUPPORTED  # fp32 not built
    assert lib.tg_gated_attention_backward(1, *args, None, 0, None) == WORKSPACE
    assert lib.tg_gated_attention_backward(1, *args, fake, need - 4, None) == WORKSPACE
    bad = list(args)
    bad[9] = 96
    assert lib.tg_gated_attention_backward(1, *bad, fake, need, None) == UNSUPPORTED
    assert lib.tg_score_grad(fake, fake, fake, seq_array(prompts), 2, 100, fake, None) == INVALID  # n_rows short


def test_gate_rejects_before_launch(lib):
    assert lib.tg_gate_score(7, None, 10, 64, None, None, 64, None, 0.0, None, None) == INVALID
    assert lib.tg_gate_score(0, None, -1, 64, None, None, 64, None, 0.0, None, None) == INVALID
    assert lib.tg_gate_score(0, None, 10, 0, None, None, 64, None, 0.0, None, None) == INVALID
    assert lib.tg_gate_score(1, None, 10, 64, None, None, 64, None, 0.0, None, None) == INVALID  # NULLs
    assert lib.tg_gate_score(1, None, 0, 64, None, None, 64, None, 0.0, None, None) == 0  # empty: no-op


def test_compact_rejects_before_launch(lib):
    ps = [Prompt(0, 10, 0, 8, 3)]
    sa = seq_array(ps)
    assert lib.tg_compact(None, 4, sa, 1, None, 0, None, None, None, None, None) == INVALID  # m mismatch
    g = (TgGather * 1)()
    g[0] = TgGather(16, 32, 24, 32, 32)  # row_bytes not a multiple of 16
    assert lib.tg_compact(None, 5, sa, 1, g, 1, None, None, None, None, None) == UNSUPPORTED
    g[0] = TgGather(16, 32, 32, 16, 32)  # stride below row_bytes
    assert lib.tg_compact(None, 5, sa, 1, g, 1, None, None, None, None, None) == INVALID
    g[0] = TgGather(None, 32, 32, 32, 32)
    assert lib.tg_compact(None, 5, sa, 1, g, 1, None, None, None, None, None) == INVALID
    # bias requested without scores
    assert lib.tg_compact(None, 5, sa, 1, None, 0, None, None, None, ctypes.c_void_p(64), None) == INVALID
    # too many gathers
    assert lib.tg_compact(None, 5, sa, 1, g, tg.TG_MAX_GATHERS + 1, None, None, None, None, None) == INVALID


def test_attention_rejects_before_launch(lib):
    ps = [Prompt(0, 10, 0, 8, 3)]
    sa = seq_array(ps)

    def call(dt=1, hq=16, hkv=8, d=128, tau=1.2, q=None):
        return lib.tg_gated_attention(dt, q, None, None, None, None, sa, 1, hq, hkv, d, None, tau,
                                      None, None, None)

    assert call(hq=12, hkv=8) == INVALID
    assert call(hkv=0) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(tau=0.0) == INVALID
    assert call(tau=float("nan")) == INVALID
    assert call(tau=float("inf")) == INVALID
    assert call(dt=5) == INVALID
    assert call() == INVALID  # NULL tensors


def test_gate_backward_workspace_and_rejects_before_launch(lib):
    # Workspace: dZ and dZ^T in bf16 over the list padded to 64 rows, per
    # 32-row tile partials of dw2 and db1, per 256-row chunk partials of dW1,
    # each region rounded up to 256 bytes.
    def up(b):
        return (b + 255) // 256 * 256

    n, d, h, nl = 16384, 2048, 256, 2384
    pad = 2432
    need = lib.tg_gate_backward_workspace_bytes(n, d, h, nl)
    assert need == 2 * up(pad * h * 2) + 2 * up(pad // 32 * h * 4) + up(((pad + 255) // 256) * h * d * 4)
    assert lib.tg_gate_backward_workspace_bytes(n, d, h, 0) == 0
    assert lib.tg_gate_backward_workspace_bytes(n, 96, h, nl) == 0      # d_model not a multiple of 64
    assert lib.tg_gate_backward_workspace_bytes(n, d, 320, nl) == 0     # d_hidden above 256
    assert lib.tg_gate_backward_workspace_bytes(n, d, h, n + 1) == 0    # list longer than the rows
    fake = ctypes.c_void_p(4096)
    args = [fake, n, d, fake, None, fake, h, fake, fake, nl, fake, fake, fake, fake, fake]
    assert lib.tg_gate_backward(0, *args, fake, need, None) == UNSUPPORTED  # fp32 not built
    assert lib.tg_gate_backward(1, *args, None, 0, None) == WORKSPACE
    assert lib.tg_gate_backward(1, *args, fake, need - 1, None) == WORKSPACE
    bad = list(args)
    bad[8] = None  # rows NULL with a shorter list
    assert lib.tg_gate_backward(1, *bad, fake, need, None) == INVALID
    bad = list(args)
    bad[6] = 192 + 32  # d_hidden not a multiple of 64
    assert lib.tg_gate_backward(1, *bad, fake, need, None) == UNSUPPORTED
    bad = list(args)
    bad[11] = None  # d_w1
    assert lib.tg_gate_backward(1, *bad, fake, need, None) == INVALID


def test_linear_and_dense_layer_reject_before_launch(lib):
    fake = ctypes.c_void_p(4096)
    assert lib.tg_linear(0, 0, fake, 10, 64, fake, None, 128, None, fake, None) == UNSUPPORTED  # fp32
    assert lib.tg_linear(1, 3, fake, 10, 64, fake, None, 128, None, fake, None) == INVALID      # epilogue
    assert lib.tg_linear(1, 0, fake, 10, 96, fake, None, 128, None, fake, None) == UNSUPPORTED  # k % 64
    assert lib.tg_linear(1, 0, fake, 10, 64, fake, None, 192, None, fake, None) == UNSUPPORTED  # n % 128
    assert lib.tg_linear(1, 1, fake, 10, 64, fake, None, 128, None, fake, None) == INVALID      # residual missing
    assert lib.tg_linear(1, 2, fake, 10, 64, fake, None, 128, None, fake, None) == INVALID      # w_up missing
    assert lib.tg_linear(1, 0, fake, 0, 64, None, None, 128, None, None, None) == OK            # nothing to do
    w = tg._lib.TgDenseWeights(2048, 16, 8, 128, 6144, 1e-6, 1e6, 1.2, *([4096] * 10))
    prompts = [Prompt(0, 100, 0, 90, 40)]
    m = 50
    need = lib.tg_dense_layer_workspace_bytes(seq_array(prompts), 1, ctypes.byref(w))
    up = lambda b: (b + 255) // 256 * 256
    assert need == sum(up(m * e * 2) for e in (2048, 4096, 2048, 1024, 1024, 2048, 2048, 6144))
    for field, bad, code in (("head_dim", 96, UNSUPPORTED), ("hkv", 3, INVALID), ("d_ff", 100, UNSUPPORTED),
                             ("d_model", 2000, UNSUPPORTED), ("tau", 0.0, INVALID), ("rope_theta", 1.0, INVALID)):
        wb = tg._lib.TgDenseWeights(2048, 16, 8, 128, 6144, 1e-6, 1e6, 1.2, *([4096] * 10))
        setattr(wb, field, bad)
        assert lib.tg_dense_layer_workspace_bytes(seq_array(prompts), 1, ctypes.byref(wb)) == 0
        assert lib.tg_dense_layer(1, fake, fake, fake, seq_array(prompts), 1, ctypes.byref(wb), fake, None, None,
                                  fake, need, None) == code, field
    assert lib.tg_dense_layer(1, fake, fake, fake, seq_array(prompts), 1, ctypes.byref(w), fake, None, None,
                              fake, need - 1, None) == WORKSPACE
    assert lib.tg_dense_layer(0, fake, fake, fake, seq_array(prompts), 1, ctypes.byref(w), fake, None, None,
                              fake, need, None) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        tg.tg_gate_score(x, torch.zeros(128, 64), torch.zeros(128))


def test_product_never_touches_oracle():
    pkg = os.path.join(ROOT, "learned_token_pruning_layer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), f
                assert "oracle" not in src or f.endswith(".py") is False or "import oracle" not in src, f


def test_layer_rejects_host_tensors():
    """The preallocated layer validates its inputs before touching the library:
    host tensors are refused (there is no CPU path)."""
    import torch
    from learned_token_pruning_layer_amd.layer import GatedPrefillLayer
    x = torch.zeros(8, 64)
    with pytest.raises(ValueError):
        GatedPrefillLayer(x, torch.zeros(4, 64), torch.zeros(4), [], [], 4, 2, 64)


def test_noalloc_decode_refuses_beyond_its_scratch(lib):
    """The allocation-free decode call checks its static scratch's size on the host,
    before any HIP call: more partials than TG_DECODE_SCRATCH_BYTES hold is refused."""
    from learned_token_pruning_layer_amd._lib import kv_seq_array
    segs = [(i << 20, 1 << 20, 4) for i in range(64)]  # 64 caches of 2^20 rows, 8 query slots
    sa = kv_seq_array(segs)
    need = lib.tg_decode_workspace_bytes(sa, len(segs), 16, 8, 128)
    assert need > (16 << 20)
    fake = ctypes.c_void_p(4096)
    st = lib.tg_decode_attention_noalloc(1, fake, fake, fake, fake, fake, sa, len(segs), 16, 8, 128, fake, 1.2, fake,
                                         None, None)
    assert st == 3
    assert b"static scratch" in lib.tg_last_error()
    # an invalid table is still reported as such first
    assert lib.tg_decode_attention_noalloc(1, fake, fake, fake, fake, fake, kv_seq_array([(0, 3, 4)]), 1, 16, 8, 128,
                                           fake, 1.0, fake, None, None) == 1


def test_check_positions_and_large_decode_tables_on_host(lib):
    """Host-side checks of the position check and of decode calls over more than
    64 sequences (their workspace covers the largest launch group)."""
    from learned_token_pruning_layer_amd._lib import kv_seq_array
    sa = seq_array([Prompt(0, 10, 0, 8, 3)])
    assert lib.tg_check_positions(None, sa, 1, None, None) == INVALID       # n_bad NULL
    assert lib.tg_check_positions(None, sa, 1, ctypes.c_void_p(64), None) == INVALID  # pos NULL with rows
    # 300 sequences: five launch groups; the workspace is that of the largest group
    segs = [(i * 1000, 1000, 1) for i in range(300)]
    many = lib.tg_decode_workspace_bytes(kv_seq_array(segs), len(segs), 16, 8, 128)
    one_group = lib.tg_decode_workspace_bytes(kv_seq_array(segs[:64]), 64, 16, 8, 128)
    assert many > 0 and one_group > 0
    # a bad sequence anywhere in the call is refused before anything is enqueued
    bad = segs[:200] + [(0, 3, 4)] + segs[200:]
    fake = ctypes.c_void_p(4096)
    assert lib.tg_decode_attention(1, fake, fake, fake, fake, fake, kv_seq_array(bad), len(bad), 16, 8, 128, fake,
                                   1.0, fake, None, fake, 1 << 30, None) == INVALID


C_CONSUMER = r"""
#include "tokengate.h"
#include <stdio.h>
#include <string.h>

int main(void) {
    /* a 100-row prompt (rows 10..89 are the document, keep 20 of them) and a
       50-row prompt that is all document, kept whole */
    tg_seq s[2] = {{0, 100, 10, 90, 20}, {100, 50, 0, 50, 50}};
    if (tg_kept_rows(s, 2) != 90) return 1;
    tg_seq bad = {0, 10, 5, 4, 0};                 /* doc_end < doc_begin */
    if (tg_kept_rows(&bad, 1) != -1) return 2;
    if (strlen(tg_last_error()) == 0) return 3;
    if (tg_select_workspace_bytes(s, 2) != 0) return 4;
    tg_seq big = {0, 40000, 0, 39000, 100};        /* above 32768 rows: needs a workspace */
    if (tg_select_workspace_bytes(&big, 1) == 0) return 5;
    if (tg_gate_score(TG_BF16, NULL, 10, 64, NULL, NULL, 128, NULL, 0.0f, NULL, NULL) != TG_ERR_INVALID_ARGUMENT)
        return 6;
    if (tg_select_topk(NULL, &big, 1, NULL, NULL, 0, NULL) == TG_OK) return 7;
    if (strlen(tg_status_string(TG_ERR_WORKSPACE)) == 0) return 8;
    puts("ok");
    return 0;
}
"""


def test_header_compiles_as_c11_and_links(tmp_path):
    """The header is plain C (C11, -Wall -Werror, gcc) and the host-side calls
    behave the same from a C program as through the binding."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    from learned_token_pruning_layer_amd._lib import LIB_PATH as so
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(so)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o", str(exe),
           "-L", libdir, "-l:" + os.path.basename(so), "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)

"""ctypes binding of libtokengate.so (the C ABI in include/tokengate.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI. torch supplies device memory and the stream. There is no
fallback: if the library is missing, or a tensor is not on a GPU, the call
raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtokengate.so")

TG_OK, TG_ERR_INVALID_ARGUMENT, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, TG_ERR_HIP = range(5)
TG_F32, TG_BF16 = 0, 1
TG_MAX_SEQS = 64
TG_MAX_GATHERS = 16

EXPORTED = (
    "tg_kept_rows", "tg_gate_score", "tg_select_workspace_bytes", "tg_select_topk", "tg_compact",
    "tg_gated_attention", "tg_decode_workspace_bytes", "tg_decode_attention",
    "tg_attention_backward_workspace_bytes", "tg_gated_attention_backward", "tg_score_grad",
    "tg_gate_backward_workspace_bytes", "tg_gate_backward", "tg_linear", "tg_dense_layer_workspace_bytes",
    "tg_dense_layer", "tg_delta_scan_workspace_bytes", "tg_gated_delta_scan", "tg_decode_attention_noalloc",
    "tg_check_positions", "tg_status_string", "tg_last_error",
)


class TokenGateError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"tokengate status {status}: {detail}")
        self.status = status
        self.detail = detail


class TgSeq(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int32), ("doc_begin", ctypes.c_int32),
                ("doc_end", ctypes.c_int32), ("k_doc", ctypes.c_int32)]


class TgKvSeq(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int32), ("n_new", ctypes.c_int32)]


class TgDenseWeights(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("tau", ctypes.c_float)] + \
               [(nm, ctypes.c_void_p) for nm in ("ln1", "wqkv", "q_norm", "k_norm", "wo", "ln2", "w_gate", "w_up",
                                                 "w_down", "gain")]


class TgGather(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("row_bytes", ctypes.c_int64),
                ("src_stride", ctypes.c_int64), ("dst_stride", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    c_int, i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    seqp = ctypes.POINTER(TgSeq)
    lib.tg_kept_rows.argtypes = [seqp, i32]
    lib.tg_kept_rows.restype = i64
    lib.tg_gate_score.argtypes = [c_int, vp, i64, i32, vp, vp, i32, vp, f32, vp, vp]
    lib.tg_gate_score.restype = c_int
    lib.tg_select_workspace_bytes.argtypes = [seqp, i32]
    lib.tg_select_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_select_topk.argtypes = [vp, seqp, i32, vp, vp, ctypes.c_size_t, vp]
    lib.tg_select_topk.restype = c_int
    lib.tg_compact.argtypes = [vp, i64, seqp, i32, ctypes.POINTER(TgGather), i32, vp, vp, vp, vp, vp]
    lib.tg_compact.restype = c_int
    lib.tg_gated_attention.argtypes = [c_int, vp, vp, vp, vp, vp, seqp, i32, i32, i32, i32, vp, f32,
                                       vp, vp, vp]
    lib.tg_gated_attention.restype = c_int
    lib.tg_attention_backward_workspace_bytes.argtypes = [seqp, i32, i32, i32, i32]
    lib.tg_attention_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_gated_attention_backward.argtypes = [c_int, vp, vp, vp, vp, vp, seqp, i32, i32, i32, i32, vp, f32,
                                                vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.tg_gated_attention_backward.restype = c_int
    lib.tg_score_grad.argtypes = [vp, vp, vp, seqp, i32, i64, vp, vp]
    lib.tg_score_grad.restype = c_int
    lib.tg_gate_backward_workspace_bytes.argtypes = [i64, i32, i32, i64]
    lib.tg_gate_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_gate_backward.argtypes = [c_int, vp, i64, i32, vp, vp, vp, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.tg_gate_backward.restype = c_int
    lib.tg_delta_scan_workspace_bytes.argtypes = [seqp, i32, i32, i32, i32]
    lib.tg_delta_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_gated_delta_scan.argtypes = [c_int, vp, vp, vp, vp, vp, seqp, i32, i32, i32, i32, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.tg_gated_delta_scan.restype = c_int
    lib.tg_linear.argtypes = [c_int, i32, vp, i64, i32, vp, vp, i32, vp, vp, vp]
    lib.tg_linear.restype = c_int
    dwp = ctypes.POINTER(TgDenseWeights)
    lib.tg_dense_layer_workspace_bytes.argtypes = [seqp, i32, dwp]
    lib.tg_dense_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_dense_layer.argtypes = [c_int, vp, vp, vp, seqp, i32, dwp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.tg_dense_layer.restype = c_int
    kvp = ctypes.POINTER(TgKvSeq)
    lib.tg_decode_workspace_bytes.argtypes = [kvp, i32, i32, i32, i32]
    lib.tg_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.tg_decode_attention.argtypes = [c_int, vp, vp, vp, vp, vp, kvp, i32, i32, i32, i32, vp, f32,
                                        vp, vp, vp, ctypes.c_size_t, vp]
    lib.tg_decode_attention.restype = c_int
    lib.tg_decode_attention_noalloc.argtypes = [c_int, vp, vp, vp, vp, vp, kvp, i32, i32, i32, i32, vp, f32, vp, vp,
                                                vp]
    lib.tg_decode_attention_noalloc.restype = c_int
    lib.tg_check_positions.argtypes = [vp, seqp, i32, vp, vp]
    lib.tg_check_positions.restype = c_int
    lib.tg_status_string.argtypes = [c_int]
    lib.tg_status_string.restype = ctypes.c_char_p
    lib.tg_last_error.argtypes = []
    lib.tg_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != TG_OK:
        lib = load()
        raise TokenGateError(status, f"{lib.tg_status_string(status).decode()}: {lib.tg_last_error().decode()}")


def seq_array(seqs: Sequence) -> ctypes.Array:
    """Prompts as a tg_seq array. Accepts objects with start, length (or
    len), doc_begin, doc_end, k_doc attributes, or 5-tuples in that order."""
    arr = (TgSeq * max(1, len(seqs)))()
    for i, s in enumerate(seqs):
        if isinstance(s, tuple) and not hasattr(s, "start"):
            start, ln, db, de, k = s
        else:
            start = s.start
            ln = getattr(s, "length", None)
            ln = s.len if ln is None else ln
            db, de, k = s.doc_begin, s.doc_end, s.k_doc
        arr[i] = TgSeq(int(start), int(ln), int(db), int(de), int(k))
    return arr


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TG_F32
    if t.dtype == torch.bfloat16:
        return TG_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def tg_kept_rows(seqs: Sequence) -> int:
    lib = load()
    m = lib.tg_kept_rows(seq_array(seqs), len(seqs))
    if m < 0:
        raise TokenGateError(TG_ERR_INVALID_ARGUMENT, lib.tg_last_error().decode())
    return int(m)


def tg_gate_score(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, b1: Optional[torch.Tensor] = None,
                  b2: float = 0.0, scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """scores[r] = w2 . SiLU(W1 x_r + b1) + b2 (fp32 [N])."""
    lib = load()
    for t, nm in ((x, "x"), (w1, "w1"), (w2, "w2")):
        _dev(t, nm)
    n, d = x.shape
    h = w1.shape[0]
    if w1.shape != (h, d) or w2.numel() != h or w1.dtype != x.dtype or w2.dtype != x.dtype:
        raise ValueError("w1 must be [H, d] and w2 [H], same dtype as x")
    if b1 is not None:
        _dev(b1, "b1")
        if b1.numel() != h or b1.dtype != x.dtype:
            raise ValueError("b1 must be [H], same dtype as x")
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=x.device)
    _check(lib.tg_gate_score(_dtype_code(x), x.data_ptr(), n, d, w1.data_ptr(), _ptr(b1), h, w2.data_ptr(),
                             float(b2), scores.data_ptr(), _stream(stream)))
    return scores


def tg_select_topk(scores: torch.Tensor, seqs: Sequence, kept_idx: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Kept packed row ids (int32 [M]), ascending within each prompt."""
    lib = load()
    _dev(scores, "scores")
    if scores.dtype != torch.float32:
        raise ValueError("scores must be fp32")
    sa = seq_array(seqs)
    m = tg_kept_rows(seqs)
    if kept_idx is None:
        kept_idx = torch.empty(m, dtype=torch.int32, device=scores.device)
    ws_bytes = lib.tg_select_workspace_bytes(sa, len(seqs))
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.tg_select_topk(scores.data_ptr(), sa, len(seqs), kept_idx.data_ptr(), _ptr(workspace),
                              ws_have, _stream(stream)))
    return kept_idx


def tg_compact(kept_idx: torch.Tensor, seqs: Sequence, tensors: Sequence[torch.Tensor] = (),
               pos: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
               want_pos: bool = True, outs: Optional[Sequence[torch.Tensor]] = None,
               pos_kept: Optional[torch.Tensor] = None, bias_kept: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[List[torch.Tensor], Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Gather kept rows of `tensors` (row = first dim), positions and bias.

    Returns (gathered, pos_kept, bias_kept); bias_kept is computed when
    `scores` is given."""
    lib = load()
    _dev(kept_idx, "kept_idx")
    m = tg_kept_rows(seqs)
    dev = kept_idx.device
    gathered = []
    garr = (TgGather * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        _dev(t, f"tensors[{i}]")
        dst = outs[i] if outs is not None else torch.empty((m,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
        row_bytes = int(math.prod(t.shape[1:])) * t.element_size()
        garr[i] = TgGather(t.data_ptr(), dst.data_ptr(), row_bytes, row_bytes, row_bytes)
        gathered.append(dst)
    if want_pos and pos_kept is None:
        pos_kept = torch.empty(m, dtype=torch.int32, device=dev)
    if scores is not None and bias_kept is None:
        bias_kept = torch.empty(m, dtype=torch.float32, device=dev)
    if pos is not None:
        _dev(pos, "pos")
    _check(lib.tg_compact(kept_idx.data_ptr(), m, seq_array(seqs), len(seqs), garr, len(tensors),
                          _ptr(pos), _ptr(pos_kept if want_pos else None), _ptr(scores),
                          _ptr(bias_kept if scores is not None else None), _stream(stream)))
    return gathered, (pos_kept if want_pos else None), (bias_kept if scores is not None else None)


def tg_gated_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bias_kept: torch.Tensor,
                       pos_kept: torch.Tensor, seqs: Sequence, gain: torch.Tensor, tau: float,
                       out: Optional[torch.Tensor] = None, want_lse: bool = False,
                       lse: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Token-gated causal attention over the kept rows.

    q [M, hq, D], k/v [M, hkv, D]; returns (out [M, hq, D], lse [hq, M] or None)."""
    lib = load()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (bias_kept, "bias_kept"), (pos_kept, "pos_kept"), (gain, "gain")):
        _dev(t, nm)
    m, hq, dh = q.shape
    hkv = k.shape[1]
    if k.shape != (m, hkv, dh) or v.shape != (m, hkv, dh):
        raise ValueError("k and v must be [M, hkv, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if bias_kept.dtype != torch.float32 or pos_kept.dtype != torch.int32 or gain.dtype != torch.float32:
        raise ValueError("bias_kept fp32, pos_kept int32, gain fp32 expected")
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((hq, m), dtype=torch.float32, device=q.device)
    sa = seq_array(seqs)
    _check(lib.tg_gated_attention(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), bias_kept.data_ptr(),
                                  pos_kept.data_ptr(), sa, len(seqs), hq, hkv, dh, gain.data_ptr(), float(tau),
                                  out.data_ptr(), _ptr(lse if want_lse else None), _stream(stream)))
    return out, (lse if want_lse else None)


def kv_seq_array(seqs: Sequence) -> ctypes.Array:
    """Decode sequences as a tg_kv_seq array: (start, len, n_new) tuples."""
    arr = (TgKvSeq * max(1, len(seqs)))()
    for i, (start, ln, n_new) in enumerate(seqs):
        arr[i] = TgKvSeq(int(start), int(ln), int(n_new))
    return arr


def tg_decode_attention(q_new: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bias: torch.Tensor,
                        pos: torch.Tensor, seqs: Sequence, gain: torch.Tensor, tau: float,
                        out: Optional[torch.Tensor] = None, want_lse: bool = False,
                        lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode over the pruned KV cache.

    q_new [R, hq, D] (the new tokens' queries, sequence by sequence);
    k/v [rows, hkv, D], bias fp32 [rows], pos int32 [rows] (the cache, the
    new tokens appended); seqs: (start, len, n_new) per sequence. Returns
    (out [R, hq, D], lse [hq, R] or None)."""
    lib = load()
    for t, nm in ((q_new, "q_new"), (k, "k"), (v, "v"), (bias, "bias"), (pos, "pos"), (gain, "gain")):
        _dev(t, nm)
    r, hq, dh = q_new.shape
    hkv = k.shape[1]
    if k.dim() != 3 or k.shape[2] != dh or v.shape != k.shape:
        raise ValueError("k and v must be [rows, hkv, D] matching q_new")
    if k.dtype != q_new.dtype or v.dtype != q_new.dtype:
        raise ValueError("q_new, k, v must share a dtype")
    if bias.dtype != torch.float32 or pos.dtype != torch.int32 or gain.dtype != torch.float32:
        raise ValueError("bias fp32, pos int32, gain fp32 expected")
    if out is None:
        out = torch.empty_like(q_new)
    if want_lse and lse is None:
        lse = torch.empty((hq, r), dtype=torch.float32, device=q_new.device)
    sa = kv_seq_array(seqs)
    ws_bytes = lib.tg_decode_workspace_bytes(sa, len(seqs), hq, hkv, dh)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q_new.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.tg_decode_attention(_dtype_code(q_new), q_new.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   bias.data_ptr(), pos.data_ptr(), sa, len(seqs), hq, hkv, dh, gain.data_ptr(),
                                   float(tau), out.data_ptr(), _ptr(lse if want_lse else None), _ptr(workspace),
                                   ws_have, _stream(stream)))
    return out, (lse if want_lse else None)


def tg_decode_attention_noalloc(q_new: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bias: torch.Tensor,
                                pos: torch.Tensor, seqs: Sequence, gain: torch.Tensor, tau: float,
                                out: Optional[torch.Tensor] = None, want_lse: bool = False,
                                lse: Optional[torch.Tensor] = None,
                                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """tg_decode_attention with the library's static scratch instead of a workspace
    (nothing is allocated by the call; outputs are allocated here only if not given)."""
    lib = load()
    for t, nm in ((q_new, "q_new"), (k, "k"), (v, "v"), (bias, "bias"), (pos, "pos"), (gain, "gain")):
        _dev(t, nm)
    r, hq, dh = q_new.shape
    hkv = k.shape[1]
    if k.dim() != 3 or k.shape[2] != dh or v.shape != k.shape:
        raise ValueError("k and v must be [rows, hkv, D] matching q_new")
    if k.dtype != q_new.dtype or v.dtype != q_new.dtype:
        raise ValueError("q_new, k, v must share a dtype")
    if bias.dtype != torch.float32 or pos.dtype != torch.int32 or gain.dtype != torch.float32:
        raise ValueError("bias fp32, pos int32, gain fp32 expected")
    if out is None:
        out = torch.empty_like(q_new)
    if want_lse and lse is None:
        lse = torch.empty((hq, r), dtype=torch.float32, device=q_new.device)
    _check(lib.tg_decode_attention_noalloc(_dtype_code(q_new), q_new.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           bias.data_ptr(), pos.data_ptr(), kv_seq_array(seqs), len(seqs), hq, hkv,
                                           dh, gain.data_ptr(), float(tau), out.data_ptr(),
                                           _ptr(lse if want_lse else None), _stream(stream)))
    return out, (lse if want_lse else None)


def tg_check_positions(pos_kept: torch.Tensor, seqs: Sequence, n_bad: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Number of kept rows (int32 [1] on the device) whose position is below the
    previous kept row's in the same prompt; 0 means the order the attention relies on holds."""
    lib = load()
    _dev(pos_kept, "pos_kept")
    if pos_kept.dtype != torch.int32:
        raise ValueError("pos_kept must be int32")
    if n_bad is None:
        n_bad = torch.empty(1, dtype=torch.int32, device=pos_kept.device)
    _check(lib.tg_check_positions(pos_kept.data_ptr(), seq_array(seqs), len(seqs), n_bad.data_ptr(), _stream(stream)))
    return n_bad


def tg_gated_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bias_kept: torch.Tensor,
                                pos_kept: torch.Tensor, seqs: Sequence, gain: torch.Tensor, tau: float,
                                out: torch.Tensor, lse: torch.Tensor, d_out: torch.Tensor,
                                workspace: Optional[torch.Tensor] = None, stream=None,
                                grads: Optional[dict] = None) -> dict:
    """Gradients of sum(d_out * out) through token-gated attention (bf16 in,
    fp32 out): dict(dq, dk, dv, dbias, dgain, dtau). out and lse are the
    forward's results for the same inputs. `grads` may hold the output
    tensors to write (same keys, fp32, contiguous)."""
    lib = load()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (bias_kept, "bias_kept"), (pos_kept, "pos_kept"), (gain, "gain"),
                  (out, "out"), (lse, "lse"), (d_out, "d_out")):
        _dev(t, nm)
    m, hq, dh = q.shape
    hkv = k.shape[1]
    if d_out.shape != q.shape or out.shape != q.shape or lse.shape != (hq, m):
        raise ValueError("out, d_out [M, hq, D] and lse [hq, M] expected")
    dev = q.device
    f32 = torch.float32
    shapes = dict(dq=(m, hq, dh), dk=(m, hkv, dh), dv=(m, hkv, dh), dbias=(m,), dgain=(hq,), dtau=(1,))
    g = {}
    for key, shp in shapes.items():
        t = grads[key] if grads is not None else torch.empty(shp, dtype=f32, device=dev)
        _dev(t, key)
        if t.dtype != f32 or t.numel() != math.prod(shp):
            raise ValueError(f"{key} must be fp32 with {math.prod(shp)} elements")
        g[key] = t
    sa = seq_array(seqs)
    ws_bytes = lib.tg_attention_backward_workspace_bytes(sa, len(seqs), hq, hkv, dh)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=dev)
    ws_have = workspace.numel() * workspace.element_size()
    _check(lib.tg_gated_attention_backward(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           bias_kept.data_ptr(), pos_kept.data_ptr(), sa, len(seqs), hq, hkv, dh,
                                           gain.data_ptr(), float(tau), out.data_ptr(), lse.data_ptr(),
                                           d_out.data_ptr(), g["dq"].data_ptr(), g["dk"].data_ptr(),
                                           g["dv"].data_ptr(), g["dbias"].data_ptr(), g["dgain"].data_ptr(),
                                           g["dtau"].data_ptr(), workspace.data_ptr(), ws_have, _stream(stream)))
    return g


def tg_score_grad(d_bias_kept: torch.Tensor, scores: torch.Tensor, kept_idx: torch.Tensor, seqs: Sequence,
                  d_scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """d(scores) [N] from d(bias_kept) [M]: sigmoid(-s) on kept document rows, 0 elsewhere."""
    lib = load()
    for t, nm in ((d_bias_kept, "d_bias_kept"), (scores, "scores"), (kept_idx, "kept_idx")):
        _dev(t, nm)
    n = scores.shape[0]
    if d_scores is None:
        d_scores = torch.empty(n, dtype=torch.float32, device=scores.device)
    _check(lib.tg_score_grad(d_bias_kept.data_ptr(), scores.data_ptr(), kept_idx.data_ptr(), seq_array(seqs),
                             len(seqs), n, d_scores.data_ptr(), _stream(stream)))
    return d_scores


def tg_gate_backward(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, d_scores: torch.Tensor,
                     rows: Optional[torch.Tensor] = None, b1: Optional[torch.Tensor] = None,
                     d_x: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None, grads: Optional[dict] = None) -> dict:
    """Gradients of sum_r d_scores[r] * scores[r] through the gate MLP over the
    listed rows (every row if rows is None): dict(dw1 [H, d], db1 [H], dw2 [H],
    db2 [1]) in fp32, plus dx when d_x (fp32 [N, d], added to) is given.
    `grads` may hold the output tensors to write (same keys)."""
    lib = load()
    for t, nm in ((x, "x"), (w1, "w1"), (w2, "w2"), (d_scores, "d_scores")):
        _dev(t, nm)
    n, d = x.shape
    h = w1.shape[0]
    if w1.shape != (h, d) or w2.numel() != h or w1.dtype != x.dtype or w2.dtype != x.dtype:
        raise ValueError("w1 must be [H, d] and w2 [H], same dtype as x")
    if d_scores.dtype != torch.float32 or d_scores.numel() != n:
        raise ValueError("d_scores must be fp32 [N]")
    if b1 is not None:
        _dev(b1, "b1")
    if rows is not None:
        _dev(rows, "rows")
        if rows.dtype != torch.int32:
            raise ValueError("rows must be int32")
    if d_x is not None:
        _dev(d_x, "d_x")
        if d_x.dtype != torch.float32 or d_x.shape != (n, d):
            raise ValueError("d_x must be fp32 [N, d]")
    n_list = n if rows is None else rows.numel()
    f32 = torch.float32
    shapes = dict(dw1=(h, d), db1=(h,), dw2=(h,), db2=(1,))
    g = {}
    for key, shp in shapes.items():
        t = grads[key] if grads is not None else torch.empty(shp, dtype=f32, device=x.device)
        _dev(t, key)
        if t.dtype != f32 or t.numel() != math.prod(shp):
            raise ValueError(f"{key} must be fp32 with {math.prod(shp)} elements")
        g[key] = t
    ws_need = lib.tg_gate_backward_workspace_bytes(n, d, h, n_list)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=x.device)
    _check(lib.tg_gate_backward(_dtype_code(x), x.data_ptr(), n, d, w1.data_ptr(), _ptr(b1), w2.data_ptr(), h,
                                d_scores.data_ptr(), _ptr(rows), n_list, _ptr(d_x), g["dw1"].data_ptr(),
                                g["db1"].data_ptr(), g["dw2"].data_ptr(), g["db2"].data_ptr(),
                                workspace.data_ptr(), workspace.numel(), _stream(stream)))
    if d_x is not None:
        g["dx"] = d_x
    return g


LINEAR_STORE, LINEAR_RESIDUAL, LINEAR_SWIGLU = 0, 1, 2


def tg_linear(x: torch.Tensor, w: torch.Tensor, residual: Optional[torch.Tensor] = None,
              w_up: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bf16 out = x W^T (+ residual), or SiLU(x W^T) * (x W_up^T) when w_up is given."""
    lib = load()
    _dev(x, "x")
    _dev(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if w.shape != (n, k) or (w_up is not None and w_up.shape != (n, k)):
        raise ValueError("weights must be [n, k]")
    epi = LINEAR_SWIGLU if w_up is not None else (LINEAR_RESIDUAL if residual is not None else LINEAR_STORE)
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    _check(lib.tg_linear(_dtype_code(x), epi, x.data_ptr(), m, k, w.data_ptr(), _ptr(w_up), n, _ptr(residual),
                         out.data_ptr(), _stream(stream)))
    return out


def dense_weights(w: dict, d_model: int, hq: int, hkv: int, head_dim: int) -> TgDenseWeights:
    """The C descriptor of a layer's weights (dict of device tensors plus tau, eps, theta)."""
    for nm in ("ln1", "wqkv", "q_norm", "k_norm", "wo", "ln2", "w_gate", "w_up", "w_down", "gain"):
        _dev(w[nm], nm)
    return TgDenseWeights(d_model, hq, hkv, head_dim, int(w["w_gate"].shape[0]), float(w["eps"]),
                          float(w["theta"]), float(w["tau"]),
                          *[w[nm].data_ptr() for nm in ("ln1", "wqkv", "q_norm", "k_norm", "wo", "ln2", "w_gate",
                                                        "w_up", "w_down", "gain")])


def tg_dense_layer(h: torch.Tensor, bias_kept: torch.Tensor, pos_kept: torch.Tensor, seqs: Sequence, w: dict,
                   hq: int, hkv: int, head_dim: int, out: Optional[torch.Tensor] = None, want_kv: bool = False,
                   workspace: Optional[torch.Tensor] = None, stream=None, k_out: Optional[torch.Tensor] = None,
                   v_out: Optional[torch.Tensor] = None):
    """One above-gate decoder layer over the kept rows h [M, d] (bf16); returns out [M, d],
    or (out, k, v) with the layer's keys and values [M, hkv, D] when want_kv."""
    lib = load()
    for t, nm in ((h, "h"), (bias_kept, "bias_kept"), (pos_kept, "pos_kept")):
        _dev(t, nm)
    m, d = h.shape
    desc = dense_weights(w, d, hq, hkv, head_dim)
    sa = seq_array(seqs)
    if out is None:
        out = torch.empty_like(h)
    k = v = None
    if want_kv:
        k = k_out if k_out is not None else torch.empty((m, hkv, head_dim), dtype=h.dtype, device=h.device)
        v = v_out if v_out is not None else torch.empty_like(k)
    need = lib.tg_dense_layer_workspace_bytes(sa, len(seqs), ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _check(lib.tg_dense_layer(_dtype_code(h), h.data_ptr(), bias_kept.data_ptr(), pos_kept.data_ptr(), sa, len(seqs),
                              ctypes.byref(desc), out.data_ptr(), _ptr(k), _ptr(v), workspace.data_ptr(),
                              workspace.numel(), _stream(stream)))
    return (out, k, v) if want_kv else out


def tg_gated_delta_scan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                        seqs: Sequence, state_in: Optional[torch.Tensor] = None, want_state: bool = False,
                        workspace: Optional[torch.Tensor] = None, stream=None, out: Optional[torch.Tensor] = None,
                        state_out: Optional[torch.Tensor] = None):
    """Gated delta rule over the kept rows: out bf16 [M, H, dv], plus the final states fp32
    [n_seqs, H, dv, dk] when want_state."""
    lib = load()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")):
        _dev(t, nm)
    m, nh, dk = k.shape
    dv = v.shape[2]
    if g.dtype != torch.float32 or beta.dtype != torch.float32 or g.shape != (m, nh) or beta.shape != (m, nh):
        raise ValueError("g and beta must be fp32 [M, H]")
    if state_in is not None:
        _dev(state_in, "state_in")
    sa = seq_array(seqs)
    if out is None:
        out = torch.empty((m, nh, dv), dtype=v.dtype, device=v.device)
    st = None
    if want_state:
        st = state_out if state_out is not None else torch.empty((len(seqs), nh, dv, dk), dtype=torch.float32,
                                                                 device=v.device)
    need = lib.tg_delta_scan_workspace_bytes(sa, len(seqs), nh, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=v.device)
    _check(lib.tg_gated_delta_scan(_dtype_code(v), q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                   beta.data_ptr(), sa, len(seqs), nh, dk, dv, _ptr(state_in), out.data_ptr(),
                                   _ptr(st), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return (out, st) if want_state else out

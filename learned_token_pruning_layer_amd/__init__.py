"""TokenGate pruned-prefill layer for MI355X (gfx950).

The four steps (gate score, top-K select, compaction, token-gated
attention), their backward (attention, bias -> score, gate MLP), the full
above-gate decoder layer, the gated delta rule of a Gated-DeltaNet layer over
the kept rows and decode over the pruned KV cache are HIP kernels behind the C ABI in
include/tokengate.h; this package is the thin ctypes binding over it
(argument marshalling only).
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    TG_BF16,
    TG_F32,
    TG_MAX_GATHERS,
    TG_MAX_SEQS,
    TokenGateError,
    load,
    seq_array,
    kv_seq_array,
    tg_check_positions,
    tg_compact,
    tg_decode_attention,
    tg_decode_attention_noalloc,
    tg_dense_layer,
    tg_gate_backward,
    tg_gate_score,
    tg_gated_attention,
    tg_gated_attention_backward,
    tg_gated_delta_scan,
    tg_kept_rows,
    tg_linear,
    tg_score_grad,
    tg_select_topk,
)
from .budget import PromptSpec, doc_budget, pack_prompts, prompt_with_budget  # noqa: F401
from .layer import GatedPrefillLayer  # noqa: F401

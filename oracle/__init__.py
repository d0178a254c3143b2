"""fp64 CPU oracle for the TokenGate pruned-prefill layer (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package; the HIP library never does.
"""

from .tokengate import (  # noqa: F401
    compact,
    decode_attention,
    dense_layer,
    gate_backward,
    gate_scores,
    gated_attention,
    gated_attention_backward,
    gated_delta_scan,
    gated_prefill,
    kept_rows,
    linear,
    logsigmoid,
    prompt_of_rows,
    rms_norm,
    rope,
    score_grad,
    select_topk,
    sigmoid,
    swiglu,
    silu,
)

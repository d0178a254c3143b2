"""Per-call pruning budget and document span -> prompt descriptors.

The pages give the user-facing side of the method this way (spke.com
article, section "Wie wird TokenGate implementiert?"): the budget of kept
prefill tokens is an argument of each generation call, and a placeholder in
the prompt template marks the document, the only part that may be pruned (the
question is always kept: same article, section "Wie hat TokenGate das
Pruning von Tokens verstanden?"). The C ABI takes the number of kept document
rows per prompt (`k_doc`). The budget here counts every kept row of a prompt,
so the document keeps what is left after the rows outside it:
    k_doc = clamp(max_kept_prefill_tokens - n_outside_doc, 0, n_doc).
A budget below the rows outside the document keeps no document row; those
rows are kept anyway, so the prompt then keeps more rows than the budget.
"""

from __future__ import annotations

from typing import List, NamedTuple, Sequence, Union


class PromptSpec(NamedTuple):
    """One packed prompt as the C ABI's tg_seq: rows [start, start + length),
    document rows [start + doc_begin, start + doc_end), k_doc of them kept."""

    start: int
    length: int
    doc_begin: int
    doc_end: int
    k_doc: int


def doc_budget(length: int, doc_begin: int, doc_end: int, max_kept_prefill_tokens: int) -> int:
    """Kept document rows of a prompt for a budget on all its kept rows."""
    if not (0 <= doc_begin <= doc_end <= length):
        raise ValueError(f"document span [{doc_begin}, {doc_end}) outside a prompt of {length} rows")
    if max_kept_prefill_tokens < 0:
        raise ValueError("max_kept_prefill_tokens must be >= 0")
    n_doc = doc_end - doc_begin
    return max(0, min(n_doc, int(max_kept_prefill_tokens) - (length - n_doc)))


def prompt_with_budget(start: int, length: int, doc_begin: int, doc_end: int,
                       max_kept_prefill_tokens: int) -> PromptSpec:
    """The prompt descriptor for one prompt and one budget."""
    return PromptSpec(int(start), int(length), int(doc_begin), int(doc_end),
                      doc_budget(length, doc_begin, doc_end, max_kept_prefill_tokens))


def pack_prompts(parts: Sequence[Sequence[int]],
                 max_kept_prefill_tokens: Union[int, Sequence[int]]) -> List[PromptSpec]:
    """Packs prompts given as (rows before the document, document rows, rows
    after it), i.e. the token counts around the placeholder, one after the
    other; the budget is one number for all prompts or one per prompt."""
    budgets = ([max_kept_prefill_tokens] * len(parts) if isinstance(max_kept_prefill_tokens, int)
               else list(max_kept_prefill_tokens))
    if len(budgets) != len(parts):
        raise ValueError("one budget per prompt")
    out, start = [], 0
    for (pre, doc, post), b in zip(parts, budgets):
        if min(pre, doc, post) < 0:
            raise ValueError("row counts must be >= 0")
        length = pre + doc + post
        out.append(prompt_with_budget(start, length, pre, pre + doc, b))
        start += length
    return out

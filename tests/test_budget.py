"""Per-call budget -> k_doc mapping (host only)."""

import pytest

import learned_token_pruning_layer_amd as tg


def test_doc_budget_clamps_to_the_document():
    # 100 rows, document [10, 90): 20 rows outside it
    assert tg.doc_budget(100, 10, 90, 50) == 30
    assert tg.doc_budget(100, 10, 90, 20) == 0
    assert tg.doc_budget(100, 10, 90, 5) == 0      # below the rows outside: no document row
    assert tg.doc_budget(100, 10, 90, 100) == 80
    assert tg.doc_budget(100, 10, 90, 10 ** 9) == 80
    assert tg.doc_budget(64, 0, 0, 10) == 0         # no document
    with pytest.raises(ValueError):
        tg.doc_budget(100, 10, 90, -1)
    with pytest.raises(ValueError):
        tg.doc_budget(100, 50, 40, 10)


@pytest.mark.parametrize("budget", [0, 1, 255, 256, 300, 4095, 4352, 10 ** 6])
def test_kept_rows_follow_the_budget(budget):
    # kept rows = max(budget, rows outside the document), at most the prompt
    p = tg.prompt_with_budget(0, 4352, 0, 4096, budget)
    assert tg.tg_kept_rows([p]) == min(max(budget, 256), 4352)


def test_pack_prompts_places_the_document_and_packs():
    ps = tg.pack_prompts([(3, 100, 7), (0, 50, 20), (5, 0, 5)], [60, 30, 4])
    assert ps == [tg.PromptSpec(0, 110, 3, 103, 50), tg.PromptSpec(110, 70, 0, 50, 10),
                  tg.PromptSpec(180, 10, 5, 5, 0)]
    assert tg.tg_kept_rows(ps) == 60 + 30 + 10
    assert tg.pack_prompts([(1, 2, 3)], 4) == [tg.PromptSpec(0, 6, 1, 3, 0)]
    with pytest.raises(ValueError):
        tg.pack_prompts([(1, 2, 3), (1, 1, 1)], [5])

"""The naive score-matrix size rule against the table the pages print."""

import json
import os

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "naive_score_matrix_table.json")


def _printed_precision(x):
    # the table rounds to two or three significant digits
    return 0.05 * x if x < 10 else 0.025 * x


def test_naive_score_table_matches_pages():
    table = json.load(open(GOLDEN))
    heads = table["heads_per_layer"]
    bpe = table["bytes_per_element"]
    for row in table["rows"]:
        n = row["context"]
        assert abs(n * n - row["scores_per_head"]) <= 0.01 * row["scores_per_head"]
        per_head = oracle.naive_score_bytes(n, 1, bpe)
        per_layer = oracle.naive_score_bytes(n, heads, bpe)
        assert abs(per_head - row["per_head_bytes"]) <= 0.05 * row["per_head_bytes"], row
        assert abs(per_layer - row["per_layer_bytes"]) <= 0.05 * row["per_layer_bytes"], row


def test_long_context_head_is_2gib_bf16():
    # 32768 tokens: 2 GiB of bf16 scores per head, never allocated by the kernels
    assert oracle.naive_score_bytes(32768) == 2 * 1024 ** 3

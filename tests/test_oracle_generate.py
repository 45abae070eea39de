"""Pins for the oracle's generation pieces: embedding rows, the first-argmax rule and the
greedy head's equivalence between exact sums and dequantised logits."""
import numpy as np

import oracle
from ternary_weight_matmul_amd import synth


def test_embed_rows_and_out_of_range_ids():
    table = np.arange(12, dtype=np.float32).reshape(4, 3)
    out = oracle.embed(np.array([2, 0, 4, -1, 3]), table)
    assert out.tolist() == [[6, 7, 8], [0, 1, 2], [0, 0, 0], [0, 0, 0], [9, 10, 11]]


def test_first_argmax_takes_the_smallest_index_of_a_tie():
    acc = np.array([[3, 7, 7, 1], [-5, -5, -9, -5], [0, 0, 0, 0], [1, 2, 3, 9]], dtype=np.int32)
    assert oracle.first_argmax(acc).tolist() == [1, 0, 0, 3]


def test_greedy_token_is_the_largest_logit():
    """dq > 0 per row, so ordering the exact sums orders the logits; where the largest logit is
    unique the token is its index."""
    g = synth.rng(51)
    x = g.standard_normal((6, 64)).astype(np.float32)
    w = (g.standard_normal((500, 64)) * 0.02).astype(np.float32)
    t, mu = oracle.ternarize(w)
    r = oracle.greedy_head(x, t, mu)
    for row in range(6):
        y = r["y"][row]
        top = np.flatnonzero(y == y.max())
        assert r["tokens"][row] == top[0]
        assert r["acc"][row, r["tokens"][row]] == r["acc"][row].max()

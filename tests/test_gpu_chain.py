"""Chained parity on the tiny CSA prefill: compressor -> indexer -> Top-k ->
sparse MQA (and C128A -> HCA), GPU chain against the oracle chain."""
import pytest

import chain

pytestmark = pytest.mark.gpu


def test_tiny_chain_all_rows():
    x = chain.inputs()
    g = chain.run_gpu(x)
    o = chain.run_oracle(x)
    rep = chain.compare(g, o, x=x)
    assert rep["topk_rows_equal"] >= 250


def test_tiny_chain_with_rope():
    """The same chain with partial RoPE (64 dims) through every stage."""
    x = chain.inputs()
    g = chain.run_gpu(x, rope=64)
    o = chain.run_oracle(x, rope=64)
    rep = chain.compare(g, o, x=x, rope=64)
    assert rep["topk_rows_equal"] >= 250

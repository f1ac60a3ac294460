"""The per-sequence KV sizes printed in "DeepSeek V4 结构速览" (KV cache 账)
reproduce from the compressed entry layout."""
import json
import os

from oracle import kv_accounting as ka

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    with open(os.path.join(GOLDEN, "kv_accounting.json")) as f:
        return json.load(f)


def test_v32_style_cache():
    g = _g()
    assert ka.v32_bytes_per_token_layer() == g["v32_bytes_per_token_layer"]
    gib = ka.v32_sequence_bytes(layers=g["v32_layers"]) / ka.GiB
    assert abs(gib - g["v32_sequence_GiB_printed"]) < 0.05
    assert gib == 83.875


def test_v4pro_layers_and_total():
    g = _g()
    assert ka.csa_layer_bytes() == g["v4pro_csa_layer_MiB"] * ka.MiB
    assert ka.hca_layer_bytes() == g["v4pro_hca_layer_MiB"] * ka.MiB
    total = ka.v4_sequence_bytes() / ka.GiB
    assert abs(total - g["v4pro_sequence_GiB_printed"]) < 0.005
    saving = ka.v32_sequence_bytes() / ka.v4_sequence_bytes()
    assert abs(saving - g["saving_factor_printed"]) < 0.05


def test_entry_counts_at_1m():
    g = _g()
    n4 = 2 ** 20 // 4
    assert abs(n4 - g["c4a_entries_at_1M_printed_approx"]) / n4 < 0.05
    assert 2 ** 20 // 128 == g["c128a_entries_at_1M_max"]

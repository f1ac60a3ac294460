"""KV-cache size accounting for the compressed cache layout.

Test infrastructure only (see the package docstring).

"DeepSeek V4 结构速览" (KV cache 账) prints per-sequence sizes at 1M
context: a V3.2-style cache of 1408 B per layer per token, about 83.9 GiB
over 61 layers; and for V4-Pro 320 MiB per CSA layer (compressed KV entries
plus indexer entries), 8 MiB per HCA layer, about 9.62 GiB in total, about
8.7x smaller.  The byte counts and entry counts inside those sentences were
lost in extraction.

Readings that reproduce every printed figure:

* Elements are 2 bytes (bf16).  A V3.2 token stores a 576-d latent and a
  128-d indexer key: (576 + 128) * 2 = 1408 B.
* A C4A entry stores a 512-d latent and a 128-d indexer key; a C128A entry
  stores a 512-d latent.  1M tokens give 2^20 / 4 C4A entries and
  2^20 / 128 C128A entries ("DeepSeek V4 结构速览", 核心设计).
* V4-Pro has 61 layers split into 30 CSA and 31 HCA layers (the split is not
  printed; it is the one that reproduces the 9.62 GiB total).
"""
from __future__ import annotations

MiB = 2 ** 20
GiB = 2 ** 30


def v32_bytes_per_token_layer(latent_dim: int = 576, index_dim: int = 128, elem: int = 2) -> int:
    return (latent_dim + index_dim) * elem


def v32_sequence_bytes(tokens: int = 2 ** 20, layers: int = 61) -> int:
    return v32_bytes_per_token_layer() * tokens * layers


def csa_layer_bytes(tokens: int = 2 ** 20, ratio: int = 4, kv_dim: int = 512,
                    index_dim: int = 128, elem: int = 2) -> int:
    return (tokens // ratio) * (kv_dim + index_dim) * elem


def hca_layer_bytes(tokens: int = 2 ** 20, ratio: int = 128, kv_dim: int = 512,
                    elem: int = 2) -> int:
    return (tokens // ratio) * kv_dim * elem


def v4_sequence_bytes(tokens: int = 2 ** 20, csa_layers: int = 30, hca_layers: int = 31) -> int:
    return csa_layers * csa_layer_bytes(tokens) + hca_layers * hca_layer_bytes(tokens)

"""KV-cache byte accounting, used to turn measured times into GB/s.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package: the product
path never imports it).

Source: "LLM 注意力与计算内核精读笔记 · 03 注意力头变体：MQA / GQA / MLA",
§3.1 and §4.1 (MQA/GQA element counts), §5.2 (MLA: latent plus decoupled RoPE
key), §7 worked examples, exercise 1 and exercise 6 (the byte function).

Per token and per layer a mechanism caches:
  MHA: keys and values of every head          -> 2 * h * d_h elements
  GQA: keys and values of g groups            -> 2 * g * d_h elements
  MQA: one shared key/value head              -> 2 * d_h elements
  MLA: one latent plus one shared RoPE key    -> d_c + d_r elements
"""
from __future__ import annotations


def kv_elements_per_token_layer(mechanism: str, h: int = 0, g: int = 0,
                                d_h: int = 0, d_c: int = 0, d_r: int = 0) -> int:
    m = mechanism.upper()
    if m == "MHA":
        return 2 * h * d_h
    if m == "GQA":
        if not 1 <= g <= h:
            raise ValueError("GQA needs 1 <= g <= h")
        return 2 * g * d_h
    if m == "MQA":
        return 2 * d_h
    if m == "MLA":
        return d_c + d_r
    raise ValueError(f"unknown mechanism {mechanism!r}")


def kv_bytes_per_token(mechanism: str, h: int = 0, g: int = 0, d_h: int = 0,
                       d_c: int = 0, d_r: int = 0, layers: int = 1,
                       bytes_per_elem: int = 2) -> int:
    """Bytes of KV cache one token occupies across `layers` layers."""
    return kv_elements_per_token_layer(mechanism, h, g, d_h, d_c, d_r) * layers * bytes_per_elem


def decode_step_cache_bytes(seq_lens, d_c: int, d_r: int, bytes_per_elem: int = 2) -> int:
    """Bytes one MLA decode step must read for one layer: every cached row of
    every sequence, once. One (d_c + d_r) row serves as both key and value, so
    the factor 2 of the MHA formula (separate K and V) does not apply."""
    return int(sum(int(L) for L in seq_lens)) * (d_c + d_r) * bytes_per_elem

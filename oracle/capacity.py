"""KV-cache capacity arithmetic stated on the pages (test oracle only).

* :func:`kv_cache_bytes` — two copies (keys and values) x layers x KV heads x head dim x tokens
  x bytes per value ("serving-paged-attention", section "캐시가 얼마나 큰지부터"; the formula's
  symbols were lost from the extracted text, its variable list survives and the 8B example in
  the same section fixes it).
* :func:`max_concurrent_requests` — cache bytes left after the weights divided by the bytes
  one request needs (same section).
* :func:`naive_waste_fraction` — reserving the maximum length for every request wastes
  ``1 - used / reserved`` ("LLM의 Paged Attention", section "Paged Attention, 이것이
  무엇일까요?").
* :func:`paged_waste_slots` — with fixed blocks only the last block's empty slots are wasted:
  ``ceil(L / BS) * BS - L`` ("serving-paged-attention", table under "블록으로 쪼개고 표로 잇는다").
"""
from __future__ import annotations


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, bytes_per_value: float) -> float:
    return 2 * layers * kv_heads * head_dim * tokens * bytes_per_value


def max_concurrent_requests(free_bytes: int, bytes_per_request: int) -> int:
    return free_bytes // bytes_per_request


def naive_waste_fraction(reserved_tokens: int, used_tokens: int) -> float:
    return 1.0 - used_tokens / reserved_tokens


def paged_waste_slots(length: int, block_size: int) -> int:
    return -(-length // block_size) * block_size - length

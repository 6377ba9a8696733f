"""Decode attention over a block-paged KV cache, in float64 (test oracle only).

What is computed, and where the pages define it:

* The KV cache is a pool of fixed-size blocks that need not be contiguous; each sequence's
  block table says which physical block holds its logical block i, and attention reads the
  scattered blocks through that table ("serving-paged-attention", section "블록으로 쪼개고
  표로 잇는다"; the talk summary's vLLM paragraph: logically contiguous, physically scattered).
  :func:`gather_sequence` reassembles a sequence's keys or values in logical order by exactly
  that lookup: token t lives in block ``table[t // BS]`` at offset ``t % BS``.
* Decode attends one new query per sequence over every token processed so far ("serving-paged-
  attention", section "캐시가 얼마나 큰지부터"); ``context_lens`` counts those tokens.
* Query heads share key/value heads in groups (MHA / GQA / MQA, talk summary, attention-heads
  paragraph); q head h reads KV head ``h // G`` with ``G = Hq / Hkv``.
* The result is ``softmax(scale * q K^T) V`` per (sequence, q head). The tiled online-softmax
  evaluation the talk summary describes (three running quantities kept on chip) reaches this
  same value up to rounding, so the oracle is the plain definition: scores, subtract the
  maximum, exponentiate, normalise, weight the values.

Readings where the pages are silent: the cache layout is ``[NB, Hkv, BS, D]``; a sequence of
length 0 yields a zero output; an 8-bit cache holds OCP E4M3 codes with one fp32 scale per
(physical block, KV head), dequantized as ``code * scale`` (exact in float64).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .fp8 import e4m3_to_float


def _widen(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if kv_dtype == "fp8_e4m3":
        return e4m3_to_float(x)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, length: int, *, kv_dtype: str = "f16",
                    scales: Optional[np.ndarray] = None) -> np.ndarray:
    """Logical ``[length, Hkv, D]`` float64 view of one sequence read through its block table."""
    bs = cache.shape[2]
    t = np.arange(length)
    phys = np.asarray(table_row, dtype=np.int64)[t // bs]
    x = _widen(cache[phys, :, t % bs, :], kv_dtype)  # [L, Hkv, D]
    if kv_dtype == "fp8_e4m3":
        if scales is None:
            raise ValueError("an E4M3 cache needs its per-(block, head) scales")
        x = x * np.asarray(scales, dtype=np.float64)[phys][:, :, None]
    return x


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v for a group of query rows q [G, D] over k, v [L, D] (float64)."""
    s = scale * (q @ k.T)  # [G, L]
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ v) / w.sum(axis=1, keepdims=True)


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
           context_lens: np.ndarray, scale: float, *, kv_dtype: str = "f16",
           k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
           seqs=None) -> np.ndarray:
    """Reference paged decode. Returns float64 ``[S, Hq, D]`` (rows of ``seqs`` only if given).

    ``scale`` is used as the float32 value the kernel receives, widened to float64.
    """
    num_seqs, hq, d = q.shape
    hkv = k_cache.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = hq // hkv
    sigma = float(np.float32(scale))
    seqs = range(num_seqs) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), hq, d), dtype=np.float64)
    for i, b in enumerate(seqs):
        length = int(context_lens[b])
        if length == 0:
            continue
        kk = gather_sequence(k_cache, block_tables[b], length, kv_dtype=kv_dtype, scales=k_scale)
        vv = gather_sequence(v_cache, block_tables[b], length, kv_dtype=kv_dtype, scales=v_scale)
        qb = q[b].astype(np.float64)
        for kvh in range(hkv):
            rows = slice(kvh * g, (kvh + 1) * g)
            out[i, rows] = attend(qb[rows], kk[:, kvh, :], vv[:, kvh, :], sigma)
    return out


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
            context_lens: np.ndarray, query_start: np.ndarray, scale: float, *,
            kv_dtype: str = "f16", k_scale: Optional[np.ndarray] = None,
            v_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal attention of a chunk of new tokens per sequence over its paged cache (float64).

    Prefill builds the KV cache from the prompt with large matrix products (talk summary,
    prefill/decode paragraphs); a chunk's keys and values are appended first, then its queries
    attend. Sequence b has ``n = query_start[b+1] - query_start[b]`` query rows in ``q`` (rows
    ``query_start[b]`` ..) which are the last n of its ``L = context_lens[b]`` tokens: query j
    sits at position ``L - n + j`` and attends to positions ``0 .. L - n + j``. Returns
    ``[T, Hq, D]``; a decode step is the case n = 1.
    """
    total, hq, d = q.shape
    hkv = k_cache.shape[1]
    g = hq // hkv
    sigma = float(np.float32(scale))
    out = np.zeros((total, hq, d), dtype=np.float64)
    for b in range(len(context_lens)):
        qs, qe = int(query_start[b]), int(query_start[b + 1])
        n, length = qe - qs, int(context_lens[b])
        if n == 0:
            continue
        kk = gather_sequence(k_cache, block_tables[b], length, kv_dtype=kv_dtype, scales=k_scale)
        vv = gather_sequence(v_cache, block_tables[b], length, kv_dtype=kv_dtype, scales=v_scale)
        for j in range(n):
            pos = length - n + j
            qj = q[qs + j].astype(np.float64)
            for kvh in range(hkv):
                rows = slice(kvh * g, (kvh + 1) * g)
                out[qs + j, rows] = attend(qj[rows], kk[: pos + 1, kvh, :], vv[: pos + 1, kvh, :], sigma)
    return out

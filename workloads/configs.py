"""Seeded synthetic decode workloads shaped like the pages' examples.

Every array is drawn from ``numpy.random.default_rng(seed)`` (integers, permutations) and, for
q, K and V, from torch's CPU normal generator seeded by that stream: standard normal in fp32
rounded to fp16 (round-to-nearest-even). Physical placement follows a seeded permutation of
the pool, handed out by the host block manager in sequence-major logical order, so a sequence's
blocks are scattered. Every slot that no sequence attends to (the tail of a last block, free
blocks, and the block that padded table entries point at) is poisoned with NaN, so a read
that the masking should have excluded shows up in the output.

The shapes come from the pages: the 8B-class head shape (32 layers x 8 KV heads x dim 128 in
fp16) and 4,096-token requests ("serving-paged-attention", section "캐시가 얼마나 큰지부터"),
100 requests behind one system prompt (section "공유는 표를 베끼는 일이 된다"), answers of 30
to 900 tokens (section "미리 잡으면 대부분이 논다"), block sizes 8/16/32/64 (section "블록
크기는 어떻게 정하나"), MHA / MQA / GQA head layouts (talk summary, attention-heads paragraph)
and an 8-bit KV cache (section "실무에서 만지는 지점"). No public dataset is involved.

Nothing here computes attention; the module only produces inputs for both the oracle and the
GPU path.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from .block_manager import BlockManager
from .quant import quantize_pool

F16_NAN = np.uint16(0x7E00)

# fixed seeds per workload
SEEDS = {"tiny": 1, "8b": 2, "prefix": 3, "prefix_fork": 31, "sweep": 4, "variants": 5,
         "prefill": 6, "shard_kvhead": 7}


@dataclass
class StepInputs:
    """One decode step's cache updates, applied before attention in stream order."""

    new_k: np.ndarray  # [T, Hkv, D] fp16
    new_v: np.ndarray
    slot_mapping: np.ndarray  # [T] int64
    block_mapping: np.ndarray  # [P, 2] int32
    pre_block_tables: np.ndarray  # tables before the step (for isolation checks)
    pre_context_lens: np.ndarray


@dataclass
class DecodeCase:
    name: str
    seed: int
    q: np.ndarray  # [S, Hq, D] fp16
    k_cache: np.ndarray  # [NB, Hkv, BS, D] fp16, or uint8 E4M3 codes
    v_cache: np.ndarray
    block_tables: np.ndarray  # [S, W] int32 (entries past a sequence's blocks = pad block)
    context_lens: np.ndarray  # [S] int32
    scale: np.float32
    block_size: int
    kv_dtype: str = "f16"  # "f16" | "fp8_e4m3"
    k_scale: Optional[np.ndarray] = None  # [NB, Hkv] f32 for fp8
    v_scale: Optional[np.ndarray] = None
    pad_block: int = -1
    # logical contiguous view (what the tables resolve to), per sequence [L, Hkv, D]
    logical_k: Optional[List[np.ndarray]] = field(default=None, repr=False)
    logical_v: Optional[List[np.ndarray]] = field(default=None, repr=False)
    step: Optional[StepInputs] = None
    # shared-prefix groups: sequences [group_start[g], group_start[g+1]) share their first
    # group_prefix_blocks[g] table entries (None when the workload has no such structure)
    group_start: Optional[np.ndarray] = None
    group_prefix_blocks: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_kv_heads(self) -> int:
        return self.k_cache.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def num_blocks(self) -> int:
        return self.k_cache.shape[0]

    @property
    def kv_bytes_per_value(self) -> int:
        return 1 if self.kv_dtype == "fp8_e4m3" else 2


def softmax_scale(head_dim: int) -> np.float32:
    return np.float32(1.0 / math.sqrt(head_dim))


def normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal fp32 draws rounded to fp16 (round-to-nearest-even).

    The draws come from torch's CPU generator seeded by one integer taken from ``rng`` (about
    ten times faster than numpy's normal sampler for the gigabyte-sized pools), so every array
    is still a deterministic function of the workload seed.
    """
    seed = int(rng.integers(0, 2 ** 62))
    g = torch.Generator().manual_seed(seed)
    return torch.randn(tuple(np.atleast_1d(shape)), generator=g, dtype=torch.float32).to(torch.float16).numpy()


def nan_pool(nb: int, hkv: int, bs: int, d: int) -> np.ndarray:
    return np.full((nb, hkv, bs, d), F16_NAN, dtype=np.uint16).view(np.float16)


def scatter_sequence(cache: np.ndarray, table: Sequence[int], values: np.ndarray, start: int = 0) -> None:
    """Write logical tokens [start, start + len(values)) of one sequence into the pool."""
    bs = cache.shape[2]
    t = np.arange(start, start + values.shape[0])
    phys = np.asarray(table, dtype=np.int64)[t // bs]
    cache[phys, :, t % bs, :] = values


def _finish(name, seed, rng_q, bm: BlockManager, logical_k, logical_v, hq, d, kv_dtype,
            q=None) -> DecodeCase:
    hkv = logical_k[0].shape[1] if logical_k else 1
    bs = bm.block_size
    pad = bm.reserve(1)[0]
    k_cache = nan_pool(bm.num_blocks, hkv, bs, d)
    v_cache = nan_pool(bm.num_blocks, hkv, bs, d)
    for s, (kk, vv) in enumerate(zip(logical_k, logical_v)):
        scatter_sequence(k_cache, bm.tables[s], kk)
        scatter_sequence(v_cache, bm.tables[s], vv)
    tables = bm.block_tables(pad_id=pad)
    if q is None:
        q = normal_f16(rng_q, (len(logical_k), hq, d))
    case = DecodeCase(name=name, seed=seed, q=q, k_cache=k_cache, v_cache=v_cache,
                      block_tables=tables, context_lens=bm.context_lens(), scale=softmax_scale(d),
                      block_size=bs, pad_block=pad, logical_k=logical_k, logical_v=logical_v)
    if kv_dtype == "fp8_e4m3":
        to_fp8(case, bm)
    return case


def to_fp8(case: DecodeCase, bm: BlockManager) -> None:
    """Replace the fp16 pool by E4M3 codes with per-(block, head) scales (in place)."""
    live = np.unique(np.concatenate([np.asarray(t, dtype=np.int64) for t in bm.tables if t]))
    case.k_cache, case.k_scale = quantize_pool(case.k_cache, live)
    case.v_cache, case.v_scale = quantize_pool(case.v_cache, live)
    case.kv_dtype = "fp8_e4m3"


def random_case(seed, lens, hq, hkv, d, bs, *, kv_dtype="f16", pool_factor=1.25,
                name="random", extra_width=0) -> DecodeCase:
    """General seeded case: independent sequences of the given lengths.

    Draw order: q, then K and V per sequence, then the block permutation; the values therefore
    do not depend on the block size or the pool size.
    """
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    q = normal_f16(rng, (len(lens), hq, d))
    lk, lv = [], []
    for L in lens:
        lk.append(normal_f16(rng, (L, hkv, d)))
        lv.append(normal_f16(rng, (L, hkv, d)))
    live = sum(-(-L // bs) for L in lens)
    nb = max(int(math.ceil(pool_factor * live)), live + 1)
    bm = BlockManager(nb, bs, free_order=rng.permutation(nb))
    for L in lens:
        bm.new_sequence(L)
    case = _finish(name, seed, rng, bm, lk, lv, hq, d, kv_dtype, q=q)
    if extra_width:
        w = case.block_tables.shape[1] + extra_width
        case.block_tables = bm.block_tables(seqs=range(len(lens)), width=w, pad_id=case.pad_block)
    return case


# --------------------------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------------------------
def tiny() -> DecodeCase:
    """4 sequences, lengths {1, 15, 16, 33}, 4 q / 2 KV heads, D 64, BS 16, 64-block pool."""
    seed = SEEDS["tiny"]
    rng = np.random.default_rng(seed)
    lens, hq, hkv, d, bs, nb = [1, 15, 16, 33], 4, 2, 64, 16, 64
    bm = BlockManager(nb, bs, free_order=rng.permutation(nb))
    q = normal_f16(rng, (len(lens), hq, d))
    lk, lv = [], []
    for L in lens:
        bm.new_sequence(L)
        lk.append(normal_f16(rng, (L, hkv, d)))
        lv.append(normal_f16(rng, (L, hkv, d)))
    case = _finish("tiny", seed, rng, bm, lk, lv, hq, d, "f16", q=q)
    assert case.scale == np.float32(0.125)
    return case


def eight_b(num_seqs: int = 64, ctx: int = 4096, seed: Optional[int] = None) -> DecodeCase:
    """8B-shaped single-layer decode: 64 x 4096 tokens, 32 q / 8 KV heads, D 128, BS 16, fp16,
    pool 1.25x the live blocks."""
    seed = SEEDS["8b"] if seed is None else seed
    return random_case(seed, [ctx] * num_seqs, 32, 8, 128, 16, name="8b")


def shared_prefix(fork: bool = False, num_seqs: int = 100, prefix_len: int = 512,
                  tail_range=(30, 900), block_size: int = 16) -> DecodeCase:
    """100 sequences behind one 512-token prefix (aliased block ids), private tails U{30..900},
    8B head shape, then one decode step: copy-on-write, slot-mapped append, attention.

    With ``fork=True`` every sequence is forked once before the step (parallel sampling), so
    each partially filled last block is shared by two siblings and the step issues copies:
    siblings sit at indices 2i (original) and 2i+1 (fork); appends run in index order, so the
    original copies and the fork then writes in place.
    """
    seed = SEEDS["prefix_fork" if fork else "prefix"]
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 32, 8, 128, block_size
    tails = rng.integers(tail_range[0], tail_range[1], endpoint=True, size=num_seqs)
    n_pref = prefix_len // bs
    assert n_pref * bs == prefix_len
    copies = 2 if fork else 1
    live = n_pref + copies * sum(-(-(int(t) + 1) // bs) for t in tails) + 1
    nb = int(math.ceil(1.25 * live))
    bm = BlockManager(nb, bs, free_order=rng.permutation(nb))
    prefix_blocks = bm.reserve(n_pref)
    pk = normal_f16(rng, (prefix_len, hkv, d))
    pv = normal_f16(rng, (prefix_len, hkv, d))
    lk, lv = [], []
    for t in tails:
        tk = normal_f16(rng, (int(t), hkv, d))
        tv = normal_f16(rng, (int(t), hkv, d))
        s = bm.new_sequence(prefix_len + int(t), prefix=prefix_blocks)
        lk.append(np.concatenate([pk, tk]))
        lv.append(np.concatenate([pv, tv]))
        if fork:
            bm.fork(s)
            lk.append(lk[-1])
            lv.append(lv[-1])
    n = len(lk)
    q = normal_f16(rng, (n, hq, d))
    # pool before the step
    k_cache = nan_pool(nb, hkv, bs, d)
    v_cache = nan_pool(nb, hkv, bs, d)
    scatter_sequence(k_cache, prefix_blocks, pk)
    scatter_sequence(v_cache, prefix_blocks, pv)
    for s in range(n):
        scatter_sequence(k_cache, bm.tables[s][n_pref:], lk[s][prefix_len:], start=0)
        scatter_sequence(v_cache, bm.tables[s][n_pref:], lv[s][prefix_len:], start=0)
    pre_lens = bm.context_lens()
    pre_tables_rows = [list(t) for t in bm.tables]
    # the step
    plan = bm.append_tokens(list(range(n)))
    new_k = normal_f16(rng, (n, hkv, d))
    new_v = normal_f16(rng, (n, hkv, d))
    pad = bm.reserve(1)[0]
    width = max(len(t) for t in bm.tables)
    pre_tables = np.full((n, width), pad, dtype=np.int32)
    for s, row in enumerate(pre_tables_rows):
        pre_tables[s, : len(row)] = row
    post_k = [np.concatenate([lk[s], new_k[s: s + 1]]) for s in range(n)]
    post_v = [np.concatenate([lv[s], new_v[s: s + 1]]) for s in range(n)]
    case = DecodeCase(
        name="prefix_fork" if fork else "prefix", seed=seed, q=q, k_cache=k_cache,
        v_cache=v_cache, block_tables=bm.block_tables(width=width, pad_id=pad),
        context_lens=bm.context_lens(), scale=softmax_scale(d), block_size=bs, pad_block=pad,
        logical_k=post_k, logical_v=post_v,
        step=StepInputs(new_k=new_k, new_v=new_v, slot_mapping=plan.slot_mapping,
                        block_mapping=plan.block_mapping, pre_block_tables=pre_tables,
                        pre_context_lens=pre_lens))
    case.prefix_blocks = prefix_blocks  # type: ignore[attr-defined]
    case.group_start = np.array([0, n], dtype=np.int32)
    case.group_prefix_blocks = np.array([n_pref], dtype=np.int32)
    return case


def prefix_groups(seed, groups, hq, hkv, d, bs, *, kv_dtype="f16",
                  name="prefix_groups") -> DecodeCase:
    """Sequences in groups behind shared prefixes ("serving-paged-attention", section "공유는
    표를 베끼는 일이 된다"). ``groups`` lists ``(members, prefix_tokens, (tail_lo, tail_hi))``:
    the group's members alias one prefix of ``prefix_tokens`` tokens (a multiple of the block
    size; 0 = nothing shared) and each has a private tail of U{tail_lo..tail_hi} tokens.

    Draw order: tail lengths, then per group the prefix K/V and each member's tail K/V, then the
    block permutation's use as blocks are taken in group order."""
    rng = np.random.default_rng(seed)
    tails = [rng.integers(lo, hi, endpoint=True, size=m) for m, _, (lo, hi) in groups]
    live = 1 + sum(pt // bs + sum(-(-int(t) // bs) + 1 for t in tl)
                   for (_, pt, _), tl in zip(groups, tails))
    nb = int(math.ceil(1.25 * live)) + 1
    bm = BlockManager(nb, bs, free_order=rng.permutation(nb))
    lk, lv = [], []
    gstart, gblocks = [0], []
    for (m, pt, _), tl in zip(groups, tails):
        assert pt % bs == 0
        pblocks = bm.reserve(pt // bs) if pt else []
        pk = normal_f16(rng, (pt, hkv, d))
        pv = normal_f16(rng, (pt, hkv, d))
        for t in tl:
            bm.new_sequence(pt + int(t), prefix=pblocks)
            lk.append(np.concatenate([pk, normal_f16(rng, (int(t), hkv, d))]))
            lv.append(np.concatenate([pv, normal_f16(rng, (int(t), hkv, d))]))
        gstart.append(gstart[-1] + m)
        gblocks.append(pt // bs)
    case = _finish(name, seed, rng, bm, lk, lv, hq, d, kv_dtype)
    case.group_start = np.array(gstart, dtype=np.int32)
    case.group_prefix_blocks = np.array(gblocks, dtype=np.int32)
    return case


@functools.lru_cache(maxsize=1)
def _sweep_logical(num_seqs: int = 128):
    rng = np.random.default_rng(SEEDS["sweep"])
    u = rng.uniform(math.log(32), math.log(8192), size=num_seqs)
    lens = np.clip(np.round(np.exp(u)), 32, 8192).astype(np.int64)
    q = normal_f16(rng, (num_seqs, 32, 128))
    lk = [normal_f16(rng, (int(L), 8, 128)) for L in lens]
    lv = [normal_f16(rng, (int(L), 8, 128)) for L in lens]
    return lens, q, lk, lv


def sweep(block_size: int, num_seqs: int = 128) -> DecodeCase:
    """128 sequences, lengths log-uniform in [32, 8192] (one draw shared by every block size),
    32 q / 8 KV heads, D 128, fp16; placement permuted per block size."""
    assert block_size in (8, 16, 32, 64)
    lens, q, lk, lv = _sweep_logical(num_seqs)
    rng = np.random.default_rng([SEEDS["sweep"], block_size])
    live = sum(-(-int(L) // block_size) for L in lens)
    nb = int(math.ceil(1.25 * live))
    bm = BlockManager(nb, block_size, free_order=rng.permutation(nb))
    for L in lens:
        bm.new_sequence(int(L))
    case = _finish(f"sweep_bs{block_size}", SEEDS["sweep"], rng, bm, lk, lv, 32, 128, "f16", q=q)
    return case


def variant(num_kv_heads: int, kv_dtype: str = "f16", num_seqs: int = 64, ctx: int = 2048) -> DecodeCase:
    """64 x 2048 tokens, BS 16, 32 q heads over 32 (MHA), 8 (GQA) or 1 (MQA) KV heads, KV in
    fp16 or E4M3 with per-(block, head) scales. The fp8 pool quantizes the same fp16 draw."""
    assert 32 % num_kv_heads == 0
    seed = SEEDS["variants"]
    case = random_case([seed, num_kv_heads], [ctx] * num_seqs, 32, num_kv_heads, 128, 16,
                       name=f"variant_hkv{num_kv_heads}_{kv_dtype}")
    case.seed = seed
    if kv_dtype == "fp8_e4m3":
        tables = [row[: -(-int(L) // 16)] for row, L in zip(case.block_tables, case.context_lens)]
        live = np.unique(np.concatenate(tables).astype(np.int64))
        case.k_cache, case.k_scale = quantize_pool(case.k_cache, live)
        case.v_cache, case.v_scale = quantize_pool(case.v_cache, live)
        case.kv_dtype = "fp8_e4m3"
    return case


def kv_head_shard(num_seqs: int = 64, ctx: int = 4096) -> DecodeCase:
    """One GPU's share of the 8B-shaped decode under 8-way KV-head sharding: the same 64 x 4096
    tokens, BS 16, D 128, fp16, but one KV head and its 4 query heads (Hq 4, Hkv 1), so the call
    reads 1/8 of the 8B workload's KV."""
    return random_case(SEEDS["shard_kvhead"], [ctx] * num_seqs, 4, 1, 128, 16,
                       name="shard_kvhead")


# --------------------------------------------------------------------------------------------
# Prefill (a chunk of new tokens per sequence attending causally over its cache)
# --------------------------------------------------------------------------------------------
@dataclass
class PrefillCase:
    """A paged cache that already holds every sequence's chunk (the chunk is the last
    ``chunk_lens[b]`` of its ``context_lens[b]`` tokens) plus the chunk queries back to back."""

    name: str
    cache: DecodeCase  # pools, tables, context lengths, scales; its q is unused
    q: np.ndarray  # [T, Hq, D] fp16
    query_start: np.ndarray  # [S + 1] int32
    chunk_lens: np.ndarray  # [S] int32

    @property
    def num_tokens(self) -> int:
        return self.q.shape[0]

    def chunk_kv(self, b: int):
        """The chunk's own keys and values [n, Hkv, D] (fp16 draws) and their slots [n]."""
        L, n = int(self.cache.context_lens[b]), int(self.chunk_lens[b])
        t = np.arange(L - n, L)
        bs = self.cache.block_size
        slots = self.cache.block_tables[b][t // bs].astype(np.int64) * bs + t % bs
        return self.cache.logical_k[b][L - n:], self.cache.logical_v[b][L - n:], slots


def prefill_case(seed, ctx_lens, chunk_lens, hq, hkv, d, bs, *, kv_dtype="f16",
                 name="prefill") -> PrefillCase:
    """Seeded prefill case: the cache of :func:`random_case` for the full context lengths, then
    the chunk queries (one fp16 normal draw of ``[sum(chunk_lens), Hq, D]``)."""
    ctx = [int(x) for x in ctx_lens]
    chunks = np.asarray([int(x) for x in chunk_lens], dtype=np.int32)
    assert len(ctx) == len(chunks) and all(0 <= n <= L for n, L in zip(chunks, ctx))
    cache = random_case(seed, ctx, hq, hkv, d, bs, kv_dtype=kv_dtype, name=name)
    rng = np.random.default_rng([int(np.sum(np.atleast_1d(seed))), 7])
    q = normal_f16(rng, (int(chunks.sum()), hq, d))
    query_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return PrefillCase(name=name, cache=cache, q=q, query_start=query_start, chunk_lens=chunks)


def prefill_8b(num_seqs: int = 16, ctx: int = 4096, chunk: int = 1024) -> PrefillCase:
    """Chunked prefill in the 8B head shape: 16 sequences whose first 3,072 tokens are cached
    and whose next 1,024-token chunk attends causally (context 4,096 after the chunk's
    append), 32 q / 8 KV heads, D 128, BS 16, fp16."""
    return prefill_case(SEEDS["prefill"], [ctx] * num_seqs, [chunk] * num_seqs, 32, 8, 128, 16,
                        name="prefill_8b")


def by_name(name: str) -> DecodeCase:
    """Lookup used by the benchmark and tests: tiny, 8b, prefix, prefix_fork, sweep_bs{8,16,32,64},
    variant_hkv{32,8,1}_{f16,fp8_e4m3}, shard_kvhead."""
    if name == "tiny":
        return tiny()
    if name == "8b":
        return eight_b()
    if name == "prefix":
        return shared_prefix(False)
    if name == "prefix_fork":
        return shared_prefix(True)
    if name.startswith("sweep_bs"):
        return sweep(int(name[len("sweep_bs"):]))
    if name == "shard_kvhead":
        return kv_head_shard()
    if name.startswith("variant_hkv"):
        rest = name[len("variant_hkv"):]
        hkv, dt = rest.split("_", 1)
        return variant(int(hkv), dt)
    raise KeyError(name)

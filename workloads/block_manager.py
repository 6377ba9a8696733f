"""Host-side KV block manager: the caller's bookkeeping that produces kernel inputs.

This is the page pool / page table / copy-on-write bookkeeping that the pages assign to the
serving side, not to the attention kernel:

* a pool of fixed-size physical blocks with a free list, handed out on demand and returned
  when freed ("LLM의 Paged Attention: 메모리 효율성을 극대화하는 방법", section "Paged
  Attention의 핵심 원리", items 1-2; "serving-paged-attention", section "블록으로 쪼개고
  표로 잇는다");
* one block table per sequence mapping logical block i to a physical block id (same
  passages);
* sharing by aliasing: several tables hold the same physical id, counted by a per-block
  reference count ("serving-paged-attention", section "공유는 표를 베끼는 일이 된다");
* copy-on-write: before a token is written into a shared block that is still filling, that
  block is copied to a private block and the writer's table is re-pointed (same section, and
  item 3 of the first page's "핵심 원리" list);
* the token -> (page, slot) placement of "vLLM의 핵심 이해: PagedAttention", section 6
  (TokenTable / SlotAllocator), expressed as a flat slot number ``block * BS + offset``.

It emits exactly what the C-ABI calls consume: ``block_tables``, ``context_lens``,
``slot_mapping`` and the (src, dst) pair list for ``pa_copy_blocks``. It holds none of the
attention arithmetic; both the oracle side and the GPU side receive its outputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when a block is requested and the free list is empty."""


@dataclass
class AppendPlan:
    """What one decode step asks of the kernels (in stream order)."""

    block_mapping: np.ndarray  # int32 [P, 2] (src, dst) copy-on-write pairs
    slot_mapping: np.ndarray  # int64 [T] flat slot = block * BS + offset
    seq_ids: List[int]  # which sequence each appended token belongs to


@dataclass
class BlockManager:
    """Free list + reference counts + per-sequence tables over ``num_blocks`` physical blocks.

    ``free_order`` fixes the order in which free blocks are handed out (a seeded permutation
    in every workload), so physical placement is scattered but reproducible.
    """

    num_blocks: int
    block_size: int
    free_order: Optional[Sequence[int]] = None
    refcount: np.ndarray = field(init=False)
    tables: List[List[int]] = field(init=False, default_factory=list)
    lens: List[int] = field(init=False, default_factory=list)
    _free: List[int] = field(init=False)

    def __post_init__(self) -> None:
        order = list(range(self.num_blocks)) if self.free_order is None else list(self.free_order)
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        # pop() takes from the end, so store reversed to hand out order[0] first
        self._free = order[::-1]
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)

    # -- pool ---------------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        if not self._free:
            raise PoolExhausted("no free KV block left in the pool")
        blk = self._free.pop()
        assert self.refcount[blk] == 0
        self.refcount[blk] = 1
        return blk

    def reserve(self, n: int = 1) -> List[int]:
        """Take ``n`` blocks out of the pool without attaching them to a sequence."""
        return [self._take() for _ in range(n)]

    def _release(self, blk: int) -> None:
        assert self.refcount[blk] > 0
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self._free.append(blk)

    # -- sequences ------------------------------------------------------------------------
    def blocks_needed(self, length: int) -> int:
        return -(-length // self.block_size)

    def new_sequence(self, length: int, prefix: Optional[Sequence[int]] = None) -> int:
        """Create a sequence holding ``length`` tokens.

        ``prefix`` lists physical ids of full blocks to alias (shared-prefix tables point at
        one physical copy); the remaining blocks are taken from the pool.
        """
        prefix = list(prefix or [])
        if len(prefix) * self.block_size > length:
            raise ValueError("shared prefix longer than the sequence")
        for blk in prefix:
            if self.refcount[blk] <= 0:
                raise ValueError("prefix block is not live")
            self.refcount[blk] += 1
        table = prefix + [self._take() for _ in range(self.blocks_needed(length) - len(prefix))]
        self.tables.append(table)
        self.lens.append(length)
        return len(self.tables) - 1

    def fork(self, seq: int) -> int:
        """Parallel-sampling fork: the child aliases every block of the parent."""
        for blk in self.tables[seq]:
            self.refcount[blk] += 1
        self.tables.append(list(self.tables[seq]))
        self.lens.append(self.lens[seq])
        return len(self.tables) - 1

    def free_sequence(self, seq: int) -> None:
        for blk in self.tables[seq]:
            self._release(blk)
        self.tables[seq] = []
        self.lens[seq] = 0

    def append_tokens(self, seqs: Sequence[int]) -> AppendPlan:
        """Place one new token for each sequence in ``seqs`` (processed in the given order).

        For each sequence with current length ``L``: if ``L`` is a multiple of the block size a
        fresh block is attached; else, if the last block is shared (reference count > 1), it
        is copied to a fresh block (one (src, dst) pair) and the table is re-pointed; the
        token then goes to slot ``table[L // BS] * BS + L % BS`` and the length grows by one.
        """
        bs = self.block_size
        pairs: List[Tuple[int, int]] = []
        slots: List[int] = []
        for s in seqs:
            length = self.lens[s]
            table = self.tables[s]
            if length % bs == 0:
                table.append(self._take())
            else:
                last = table[-1]
                if self.refcount[last] > 1:
                    dst = self._take()
                    pairs.append((last, dst))
                    self.refcount[last] -= 1
                    table[-1] = dst
            slots.append(table[length // bs] * bs + length % bs)
            self.lens[s] = length + 1
        plan = AppendPlan(
            block_mapping=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
            slot_mapping=np.asarray(slots, dtype=np.int64),
            seq_ids=list(seqs),
        )
        check_plan(plan, bs)
        return plan

    # -- exports --------------------------------------------------------------------------
    def block_tables(self, seqs: Optional[Sequence[int]] = None, width: Optional[int] = None,
                     pad_id: int = 0) -> np.ndarray:
        seqs = range(len(self.tables)) if seqs is None else seqs
        rows = [self.tables[s] for s in seqs]
        w = max((len(r) for r in rows), default=0) if width is None else width
        out = np.full((len(rows), max(w, 1)), pad_id, dtype=np.int32)
        for i, r in enumerate(rows):
            if len(r) > w:
                raise ValueError("table wider than requested width")
            out[i, : len(r)] = r
        return out

    def context_lens(self, seqs: Optional[Sequence[int]] = None) -> np.ndarray:
        seqs = range(len(self.tables)) if seqs is None else seqs
        return np.asarray([self.lens[s] for s in seqs], dtype=np.int32)

    def waste_slots(self, seq: int) -> int:
        """Allocated-but-unused slots of one sequence: n_b * BS - L."""
        return len(self.tables[seq]) * self.block_size - self.lens[seq]


def check_plan(plan: AppendPlan, block_size: int) -> None:
    """Preconditions the kernels rely on: unique slots, distinct copy targets disjoint from
    the copy sources."""
    slots = plan.slot_mapping
    if len(np.unique(slots)) != len(slots):
        raise AssertionError("duplicate slot in one step")
    if len(plan.block_mapping):
        src, dst = plan.block_mapping[:, 0], plan.block_mapping[:, 1]
        if len(np.unique(dst)) != len(dst):
            raise AssertionError("two copies target one block")
        if np.intersect1d(src, dst).size:
            raise AssertionError("a copy target is also a copy source")

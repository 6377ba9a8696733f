"""Host-side accounting of the benchmark (no GPU): algorithmic KV bytes per call, the bytes of
one decode call, and the step inputs that rewrite each sequence's newest position, pinned to
closed forms of the workloads' shapes."""
import numpy as np

import bench
import workloads


def test_tiny_kv_bytes_closed_form():
    # 65 attended tokens x (K and V) x 2 KV heads x 64 dims x 2 bytes
    case = workloads.tiny()
    assert bench.kv_bytes(case) == 65 * 2 * 2 * 64 * 2 == 33280
    assert bench.kv_bytes(case, unique=False) == 33280
    # + q and out (4 seqs x 4 heads x 64 x 2 bytes each) + one table entry per used block
    # (1, 1, 1, 3 blocks at BS 16) + one context length per sequence
    assert bench.decode_call_bytes(case) == 33280 + 2 * 4 * 4 * 64 * 2 + 4 * 6 + 4 * 4


def test_shared_prefix_counts_the_prefix_once():
    # two groups: 3 members behind 32 shared tokens, 2 members behind nothing
    case = workloads.prefix_groups(11, [(3, 32, (5, 20)), (2, 0, (40, 60))], 8, 2, 64, 16)
    per_tok = 2 * 2 * 64 * 2
    lens = case.context_lens.astype(int)
    logical = int(lens.sum()) * per_tok
    unique = (32 + int(lens[:3].sum()) - 3 * 32 + int(lens[3:].sum())) * per_tok
    assert bench.kv_bytes(case, unique=False) == logical
    assert bench.kv_bytes(case) == unique


def test_fp8_kv_bytes_add_the_block_scales():
    case = workloads.random_case(12, [1, 16, 17], 4, 2, 64, 16, kv_dtype="fp8_e4m3")
    blocks = 1 + 1 + 2
    assert bench.kv_bytes(case) == 34 * 2 * 2 * 64 * 1 + 2 * 2 * 4 * blocks


def test_step_inputs_rewrite_the_newest_position_in_place():
    case = workloads.random_case(13, [1, 15, 16, 33, 200], 8, 2, 64, 16)
    pairs, nk, nv, slots = bench.make_step_inputs(case)
    assert pairs.shape == (0, 2)
    bs = case.block_size
    for b, L in enumerate(case.context_lens.astype(int)):
        blk, off = divmod(int(slots[b]), bs)
        assert blk == case.block_tables[b, (L - 1) // bs] and off == (L - 1) % bs
        # the row already cached there, so repeated steps keep the inputs unchanged
        assert np.array_equal(nk[b].view(np.uint16), case.k_cache[blk, :, off, :].view(np.uint16))
        assert np.array_equal(nv[b].view(np.uint16), case.v_cache[blk, :, off, :].view(np.uint16))


def test_kv_head_shard_reads_an_eighth_of_the_8b_workload():
    # the shard keeps the 8B shape's sequences, lengths, block size and head dim with one of
    # its eight KV heads (and that head's four query heads)
    shard, full = workloads.kv_head_shard(), workloads.eight_b()
    assert (shard.num_seqs, shard.head_dim, shard.block_size) == (full.num_seqs, full.head_dim,
                                                                  full.block_size)
    assert np.array_equal(shard.context_lens, full.context_lens)
    assert (shard.num_q_heads, shard.num_kv_heads) == (4, 1)
    assert bench.kv_bytes(shard) * 8 == bench.kv_bytes(full) == 1 << 30


def test_bench_measures_one_gpu_only():
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=root, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr

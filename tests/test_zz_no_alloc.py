"""pa_decode_append_noalloc, whose split-context workspace is the library's own per-GPU device
array, against pa_decode_append with a caller-allocated workspace.

Two calls in a row through the C ABI, the second with a smaller input (fewer sequences, shorter
contexts, another head layout), each after a larger one has left its partials in the array:
caches and outputs must be bit-identical to the existing entry point's (the same kernels run on
the same partitions), the appended caches must equal the oracle's append over the whole pool,
and the outputs must lie within the attention tolerance of the oracle. An E4M3 call follows.
(A call too large for the array is rejected before anything is enqueued: a CPU test.)
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_helpers import (assert_attention_close, bits, case_to_device, dev, gen, host_bits,
                            log)

pytestmark = pytest.mark.gpu


def new_rows(case, seed):
    rng = np.random.default_rng(seed)
    s, hkv, d, bs = case.num_seqs, case.num_kv_heads, case.head_dim, case.block_size
    nk = rng.standard_normal((s, hkv, d), dtype=np.float32).astype(np.float16)
    nv = rng.standard_normal((s, hkv, d), dtype=np.float32).astype(np.float16)
    slots = np.array([int(case.block_tables[b, (int(L) - 1) // bs]) * bs + (int(L) - 1) % bs
                      for b, L in enumerate(case.context_lens)], np.int64)
    return nk, nv, slots


def oracle_step(case, nk, nv, slots):
    if case.kv_dtype == "f16":
        ek, ev = oracle.kv_write(nk, nv, case.k_cache, case.v_cache, slots)
        eks = evs = None
    else:
        ek, ev, eks, evs = oracle.kv_write_fp8(nk, nv, case.k_cache, case.v_cache, case.k_scale,
                                               case.v_scale, slots)
    ref = oracle.decode(case.q, ek, ev, case.block_tables, case.context_lens, case.scale,
                        kv_dtype=case.kv_dtype, k_scale=eks, v_scale=evs)
    return ek, ev, eks, evs, ref


def compare(case, seed, pt, what):
    import paged_kv_cache_287_amd as pa

    log(f"[noalloc] {what}: S={case.num_seqs} {case.num_q_heads}q/{case.num_kv_heads}kv "
        f"D={case.head_dim} BS={case.block_size} {case.kv_dtype} partition={pt}")
    nk, nv, slots = new_rows(case, seed)
    kvt = pa.PA_KV_F16 if case.kv_dtype == "f16" else pa.PA_KV_FP8_E4M3
    need = pa.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                     case.head_dim, case.block_size,
                                     case.block_tables.shape[1] * case.block_size, kvt, pt)
    assert 0 < need <= pa.NOALLOC_SCRATCH_BYTES, need  # the library's array is in use
    g_nk, g_nv, g_slots = dev(nk), dev(nv), dev(slots)
    d_ref, d_new = case_to_device(case), case_to_device(case)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out_ref = torch.full_like(d_ref["q"], float("nan"))
    out_new = torch.full_like(d_new["q"], float("nan"))
    pa.pa_decode_append(out_ref, d_ref["q"], g_nk, g_nv, d_ref["k_cache"], d_ref["v_cache"],
                        g_slots, d_ref["block_tables"], d_ref["context_lens"], float(case.scale),
                        k_scale=d_ref["k_scale"], v_scale=d_ref["v_scale"], partition_tokens=pt,
                        workspace=ws)
    pa.pa_decode_append_noalloc(out_new, d_new["q"], g_nk, g_nv, d_new["k_cache"],
                                d_new["v_cache"], g_slots, d_new["block_tables"],
                                d_new["context_lens"], float(case.scale),
                                k_scale=d_new["k_scale"], v_scale=d_new["v_scale"],
                                partition_tokens=pt)
    torch.cuda.synchronize()
    assert torch.equal(out_new.view(torch.int16), out_ref.view(torch.int16)), \
        f"{what}: output differs from pa_decode_append"
    ek, ev, eks, evs, ref = oracle_step(case, nk, nv, slots)
    for name, e in (("k_cache", ek), ("v_cache", ev)):
        assert np.array_equal(bits(d_new[name]), host_bits(e)), f"{what}: {name} vs the oracle"
        assert torch.equal(d_new[name].view(torch.uint8), d_ref[name].view(torch.uint8)), name
    if eks is not None:
        assert np.array_equal(bits(d_new["k_scale"]), host_bits(eks))
        assert np.array_equal(bits(d_new["v_scale"]), host_bits(evs))
    assert_attention_close(out_new, ref, what)


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    big = gen(workloads.random_case, 1300, [3000, 2047, 2900, 1, 2500, 1800, 3100, 2222] * 2,
              32, 8, 128, 16, name="noalloc_big")
    small = gen(workloads.random_case, 1301, [700, 257, 900, 513], 32, 1, 64, 8,
                name="noalloc_small")
    compare(big, 1302, 256, "first call (16 seqs, GQA-4, D 128)")
    compare(small, 1303, 256, "second, smaller call (4 seqs, MQA, D 64)")
    fp8 = gen(workloads.random_case, 1304, [1200, 2000, 333], 32, 8, 128, 16,
              kv_dtype="fp8_e4m3", name="noalloc_fp8")
    compare(fp8, 1305, 256, "E4M3 call")
    compare(small, 1306, 256, "the smaller call again")


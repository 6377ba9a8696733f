#!/usr/bin/env python3
"""Benchmark of the paged decode-attention hot path on one MI355X.

One step is one decode step of the whole path over one batch: ``pa_copy_blocks`` (the step's
copy-on-write pairs, if any), ``pa_kv_write`` (one new token per sequence into its slot) and
``pa_decode`` over every attended token. Inputs are synthetic, seeded, and resident in HBM
before the timed region starts. The default workload is the 8B-shaped decode: 64 sequences x
4096 tokens, 32 query / 8 KV heads, head dim 128, block size 16, fp16 KV, blocks scattered over
a pool 1.25x the live blocks.

Prints ONE JSON line. ``value`` is KV bytes attended per second (GB/s, decimal) over whole
steps; ``roofline`` prices ``pa_decode`` (its algorithmic bytes: KV + q + out + tables) per
call against the 8 TB/s HBM peak, with the call's duration taken from HIP events recorded on
the stream the kernels run on; ``cpu_baseline`` times the float64 CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak of an MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_8b_traffic.json")
# sources of the 8B workload's decode kernel (GQA-4: the matrix-core kernel), whose measured HBM
# traffic profiles/decode_8b_traffic.json holds while they are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_287_amd", "csrc", f)
                  for f in ("decode_mfma.hip", "decode_common.hpp", "fp8_append.hpp",
                            "pa_internal.hpp")]


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_kernel_family(group: int, shared: bool) -> str:
    """Which decode kernel the library runs for G query heads per KV head (the library's rule:
    matrix-core tiles from G = 4, from G = 5 in shared-prefix decode, when the group fits one
    tile of at most 32 rows or splits evenly into such tiles; the vector-ALU kernel otherwise)."""
    if group >= (5 if shared else 4):
        if group % 16 == 0 or group % (-(-group // 32)) == 0:
            return "matrix-core decode kernel"
    return "vector-ALU decode kernel"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed ones (the first ~10 ms of back-to-back "
                         "calls after the GPU idled run ~6 %% slower on MI355X)")
    ap.add_argument("--workload", default="8b",
                    help="8b | tiny | prefix | sweep_bs{8,16,32,64} | variant_hkv{32,8,1}_{f16,fp8_e4m3}"
                         " | shard_kvhead (one GPU's share of 8b under 8-way KV-head sharding)"
                         " | prefill_8b (chunked prefill: its own JSON line in TFLOP/s)")
    ap.add_argument("--flushed-calls", type=int, default=50,
                    help="pa_decode calls timed one by one after evicting the caches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quality", action=argparse.BooleanOptionalAction, default=True,
                    help="report the E4M3-vs-fp16 error of the head-layout variants (a sample)")
    ap.add_argument("--probe-gib", type=float, default=4.0,
                    help="size of the streaming-read probe that measures attainable bandwidth (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--swap-blocks", type=int, default=1024,
                    help="blocks swapped out to pinned host memory and back for the swap figure (0 = skip)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step from a captured HIP graph instead of launching it eagerly "
                         "(measured slower on MI355X: the graph adds a fence between its nodes)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy three times: a kernel of "
                         "known traffic that hardware byte counters are scaled against")
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="split-context partition size passed to pa_decode (0 = library's choice)")
    ap.add_argument("--append", choices=["fused", "separate"], default="fused",
                    help="fused: the step's append runs inside the decode call (pa_decode_append) "
                         "wherever the step is one token per sequence at its newest position; "
                         "separate: pa_kv_write, then the decode call")
    ap.add_argument("--seq-order", choices=["longest", "natural"], default="longest",
                    help="dispatch order passed to the decode call: longest contexts first (the "
                         "host knows the lengths; no order is passed when it is the batch order) "
                         "or the batch order")
    ap.add_argument("--decode", choices=["auto", "plain", "shared_prefix"], default="auto",
                    help="decode entry point: shared_prefix reads each group's shared blocks once "
                         "(auto: whenever the workload has prefix groups)")
    return ap.parse_args()


def describe(case) -> str:
    lens = case.context_lens
    same = int(lens.min()) == int(lens.max())
    ctx = f"{int(lens[0])} tokens" if same else f"{int(lens.min())}-{int(lens.max())} tokens"
    return (f"paged decode {case.name}: {case.num_seqs} seqs x {ctx}, {case.num_q_heads}q/"
            f"{case.num_kv_heads}kv heads, head_dim {case.head_dim}, block_size {case.block_size}, "
            f"{case.kv_dtype} KV, pool {case.num_blocks} blocks")


def kv_bytes(case, unique: bool = True) -> int:
    """Algorithmic KV bytes one decode reads: every attended token's K and V for every KV head
    (shared blocks counted once when ``unique``), plus per-block scales for 8-bit caches."""
    bs, esz = case.block_size, case.kv_bytes_per_value
    per_tok = 2 * case.num_kv_heads * case.head_dim * esz
    used = {}
    total_tok = 0
    for row, L in zip(case.block_tables, case.context_lens):
        L = int(L)
        total_tok += L
        for i in range(-(-L // bs)):
            n = min(bs, L - i * bs)
            blk = int(row[i])
            used[blk] = max(used.get(blk, 0), n)
    tok = sum(used.values()) if unique else total_tok
    blocks = len(used) if unique else sum(-(-int(L) // bs) for L in case.context_lens)
    scales = 2 * case.num_kv_heads * 4 * blocks if case.kv_dtype != "f16" else 0
    return tok * per_tok + scales


def decode_call_bytes(case) -> int:
    s, hq, d = case.q.shape
    tables = sum(4 * -(-int(L) // case.block_size) for L in case.context_lens) + 4 * s
    return kv_bytes(case) + 2 * s * hq * d * 2 + tables


def make_step_inputs(case):
    """The step's cache updates. Workloads without an explicit step rewrite each sequence's
    newest token (position L - 1) in place, which keeps the inputs identical across steps."""
    import numpy as np

    if case.step is not None:
        st = case.step
        return st.block_mapping.reshape(-1, 2), st.new_k, st.new_v, st.slot_mapping
    bs = case.block_size
    ks, vs, slots = [], [], []
    for b, L in enumerate(case.context_lens):
        L = int(L)
        if L == 0:
            continue
        ks.append(case.logical_k[b][L - 1])
        vs.append(case.logical_v[b][L - 1])
        slots.append(int(case.block_tables[b, (L - 1) // bs]) * bs + (L - 1) % bs)
    return (np.zeros((0, 2), np.int32), np.stack(ks), np.stack(vs), np.asarray(slots, np.int64))


def _oracle_worker(args):
    """One process of the CPU baseline: decode its share of the sequences with the oracle, again
    and again, until its time budget is spent (BLAS limited to one thread in the process)."""
    case, seqs, budget_s = args
    import oracle

    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    per_tok = 2 * case.num_kv_heads * case.head_dim * case.kv_bytes_per_value
    done, tok_done, bytes_done = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        for b in seqs:
            oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                          case.scale, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                          v_scale=case.v_scale, seqs=[b])
            done += 1
            tok_done += int(case.context_lens[b])
            bytes_done += int(case.context_lens[b]) * per_tok
            if time.perf_counter() - t0 > budget_s:
                return done, tok_done, bytes_done, time.perf_counter() - t0


_POOL_CASE = None  # the workload, inherited by the forked oracle processes


def _pool_worker(args):
    seqs, budget_s = args
    return _oracle_worker((_POOL_CASE, seqs, budget_s))


def cpu_baseline(case, budget_s: float, max_workers: int = 16):
    """The float64 oracle on the host's cores: one process per core (at most ``max_workers``,
    the CPU share of one GPU on the measurement boxes), each with BLAS at one thread, deals the
    sequences round-robin and decodes its share until the budget is spent; then the same on one
    core for comparison. Must run before the GPU is initialised (the processes are forked)."""
    global _POOL_CASE
    import multiprocessing as mp

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, max_workers, case.num_seqs))
    share = [list(range(w, case.num_seqs, workers)) for w in range(workers)]
    _POOL_CASE = case
    multi_s = budget_s * 2 / 3
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        res = pool.map(_pool_worker, [(sh, multi_s) for sh in share])
        wall = time.perf_counter() - t0
    _POOL_CASE = None
    done = sum(r[0] for r in res)
    tok = sum(r[1] for r in res)
    byt = sum(r[2] for r in res)
    one = _oracle_worker((case, list(range(case.num_seqs)), budget_s / 3))
    return {"value": byt / wall / 1e9, "unit": "GB/s", "cores": workers, "threads": workers,
            "affinity_cores": affinity, "kind": "oracle",
            "sample": f"{done} sequence decodes of the same workload ({tok} seq-tokens) in "
                      f"{wall:.1f} s by {workers} processes with BLAS at 1 thread each "
                      f"(sequences dealt round-robin, repeated until each process's "
                      f"{multi_s:.0f} s budget ran out), float64 numpy",
            "seq_tokens_per_s": tok / wall,
            "one_core": {"value": one[2] / one[3] / 1e9, "unit": "GB/s", "cores": 1,
                         "seq_tokens_per_s": one[1] / one[3],
                         "sample": f"{one[0]} sequence decodes in {one[3]:.1f} s on one process"}}


def e4m3_quality(num_seqs: int = 4):
    """Quality of the 8-bit KV cache, reported and not gated ("serving-paged-attention", section
    "실무에서 만지는 지점": the effect of 8-bit KV on quality has to be measured on its own).
    For each head layout of the head-layout variants (64 x 2048 tokens, Hq 32, Hkv 32 / 8 / 1;
    here num_seqs sequences drawn by the same recipe), the E4M3 pool quantizes the same fp16
    draw; the oracle decodes both, and pa_decode decodes the E4M3 pool on the GPU. Errors are
    against the oracle's fp16-KV output: max |err|, and max |err| / max(|ref|, 2e-3)."""
    import numpy as np
    import torch

    import oracle
    import paged_kv_cache_287_amd as pa
    import workloads

    def dev(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.float16:
            return torch.from_numpy(x.view(np.uint16)).cuda().view(torch.float16)
        return torch.from_numpy(x).cuda()

    def errs(got, ref):
        e = np.abs(got - ref)
        return {"max_abs_err": float(e.max()),
                "max_rel_err": float((e / np.maximum(np.abs(ref), 2e-3)).max()),
                "max_err_over_max_ref": float(e.max() / np.abs(ref).max()),
                "rms_err": float(np.sqrt(np.mean(e ** 2)))}

    report = {}
    for hkv in (32, 8, 1):
        f16 = workloads.variant(hkv, "f16", num_seqs=num_seqs)
        e4 = workloads.variant(hkv, "fp8_e4m3", num_seqs=num_seqs)
        ref = oracle.decode(f16.q, f16.k_cache, f16.v_cache, f16.block_tables, f16.context_lens,
                            f16.scale)
        o8 = oracle.decode(e4.q, e4.k_cache, e4.v_cache, e4.block_tables, e4.context_lens,
                           e4.scale, kv_dtype="fp8_e4m3", k_scale=e4.k_scale, v_scale=e4.v_scale)
        out = torch.empty(e4.q.shape, dtype=torch.float16, device="cuda")
        pa.pa_decode(out, dev(e4.q), dev(e4.k_cache), dev(e4.v_cache), dev(e4.block_tables),
                     dev(e4.context_lens), float(e4.scale), k_scale=dev(e4.k_scale),
                     v_scale=dev(e4.v_scale))
        gpu = out.float().cpu().numpy().astype(np.float64)
        name = {32: "mha", 8: "gqa4", 1: "mqa"}[hkv]
        report[name] = {"oracle_e4m3_vs_oracle_f16": errs(o8, ref),
                        "gpu_e4m3_vs_oracle_f16": errs(gpu, ref)}
    report["sample"] = (f"{num_seqs} sequences x 2048 tokens per head layout (Hq 32, D 128, BS 16),"
                        f" seeded as the head-layout variants; E4M3 with one fp32 scale per"
                        f" (block, KV head)")
    return report


def prefill_flops(pc) -> int:
    """Algorithmic flops of one causal chunk attention: a query at position p multiplies with
    p + 1 keys and p + 1 values, 2 * D flops each, for every query head."""
    c = pc.cache
    total = 0
    for b in range(c.num_seqs):
        n, L = int(pc.chunk_lens[b]), int(c.context_lens[b])
        total += n * (L - n) + n * (n + 1) // 2  # sum over j < n of (L - n + j + 1)
    return 4 * c.head_dim * c.num_q_heads * total


def prefill_cpu_baseline(pc, budget_s: float):
    """Time the float64 oracle on single rows of the same workload (each row is a one-row chunk
    at its own context length) until the budget is spent."""
    import numpy as np

    import oracle

    c = pc.cache
    rng = np.random.default_rng(0)
    flops, rows = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = int(rng.integers(0, c.num_seqs))
        n, L = int(pc.chunk_lens[b]), int(c.context_lens[b])
        j = int(rng.integers(0, n))
        row = int(pc.query_start[b]) + j
        oracle.prefill(pc.q[row: row + 1], c.k_cache, c.v_cache, c.block_tables[b: b + 1],
                       np.array([L - n + j + 1], dtype=np.int32), np.array([0, 1], dtype=np.int32),
                       c.scale)
        flops += 4 * c.head_dim * c.num_q_heads * (L - n + j + 1)
        rows += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} random query rows (all heads) of the same workload, each as a "
                      f"one-row chunk, {dt:.1f} s, float64 numpy"}


def main_prefill(args):
    """Chunked prefill: one step is the chunk's append (pa_kv_write of every chunk token) and
    the causal attention of the chunk over the cache (pa_prefill)."""
    import numpy as np
    import torch

    import paged_kv_cache_287_amd as pa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    progress(f"generating workload {args.workload}")
    pc = workloads.prefill_8b()
    c = pc.cache

    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.float16:
            return torch.from_numpy(x.view(np.uint16)).cuda().view(torch.float16)
        return torch.from_numpy(x).cuda()

    parts = [pc.chunk_kv(b) for b in range(c.num_seqs)]
    g_nk = dev(np.concatenate([p[0] for p in parts]))
    g_nv = dev(np.concatenate([p[1] for p in parts]))
    g_slots = dev(np.concatenate([p[2] for p in parts]).astype(np.int64))
    q, kc, vc = dev(pc.q), dev(c.k_cache), dev(c.v_cache)
    tables, lens, qstart = dev(c.block_tables), dev(c.context_lens), dev(pc.query_start)
    out = torch.empty_like(q)
    max_q, max_ctx = int(pc.chunk_lens.max()), int(c.context_lens.max())
    stream = torch.cuda.current_stream()

    def prefill():
        pa.pa_prefill(out, q, kc, vc, tables, lens, qstart, float(c.scale), max_query_len=max_q,
                      max_context_len=max_ctx)

    def step():
        pa.pa_kv_write(g_nk, g_nv, kc, vc, g_slots)
        prefill()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n, e0.elapsed_time(e1) * 1e-3 / n

    if args.calibrate:
        progress("calibration copy: 3 x 256 MiB read + 256 MiB written")
        src = torch.ones(2 ** 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    progress(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    progress(f"timing {args.steps} steps")
    wall_step, event_step = timed(step, args.steps)
    progress(f"timing {args.steps} prefill calls")
    _, event_call = timed(prefill, args.steps)
    flops = prefill_flops(pc)
    achieved = flops / event_call / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        progress(f"oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        cpu = prefill_cpu_baseline(pc, args.cpu_seconds)
    line = {
        "metric": "paged chunked prefill: causal attention TFLOP/s, 8B-shaped, 1 GPU",
        "value": flops / wall_step / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_step * 1e3,
        "event_ms_per_step": event_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) fp16 q/K/V, scattered blocks, NaN-poisoned unused slots)",
        "config": {"workload": f"paged chunked prefill {pc.name}: {c.num_seqs} seqs, chunk "
                               f"{max_q} tokens at context {max_ctx}, {c.num_q_heads}q/"
                               f"{c.num_kv_heads}kv heads, head_dim {c.head_dim}, block_size "
                               f"{c.block_size}, {c.kv_dtype} KV",
                   "step": "kv_write(chunk) + prefill"},
        "flops_per_call": flops,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "pa_prefill (prefill_kernel)", "avg_call_us": event_call * 1e6,
                     "timing": "HIP events around the timed back-to-back pa_prefill calls"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence or by KV head with no exchange inside "
              "attention: one process per GPU, each on its own share)", file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("prefill"):
        return main_prefill(args)
    import numpy as np
    import torch

    import paged_kv_cache_287_amd as pa
    import workloads

    progress(f"generating workload {args.workload}")
    case = workloads.by_name(args.workload)
    pairs, nk, nv, slots = make_step_inputs(case)
    # the CPU baseline forks its oracle processes, so it runs before anything touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        progress(f"oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(case, args.cpu_seconds)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    def dev(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.float16:
            return torch.from_numpy(x.view(np.uint16)).cuda().view(torch.float16)
        return torch.from_numpy(x).cuda()

    q, kc, vc = dev(case.q), dev(case.k_cache), dev(case.v_cache)
    ks, vs = dev(case.k_scale), dev(case.v_scale)
    tables, lens = dev(case.block_tables), dev(case.context_lens)
    g_pairs, g_nk, g_nv, g_slots = dev(pairs.astype(np.int32)), dev(nk), dev(nv), dev(slots)
    out = torch.empty_like(q)
    max_ctx = int(case.context_lens.max())
    kvt = pa.PA_KV_F16 if case.kv_dtype == "f16" else pa.PA_KV_FP8_E4M3
    part_tokens = pa.decode_partition_tokens(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                             case.head_dim, case.block_size, max_ctx, kvt,
                                             args.partition_tokens)
    ws_bytes = pa.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                         case.head_dim, case.block_size, max_ctx, kvt, part_tokens)
    shared = case.group_start is not None if args.decode == "auto" else args.decode == "shared_prefix"
    if shared:
        assert case.group_start is not None, "this workload has no shared-prefix groups"
        # the shared-prefix call has its own automatic size (its kernel choice can differ from
        # pa_decode's): pass the requested value, 0 letting the library resolve it
        part_tokens = args.partition_tokens
        ws_bytes = pa.shared_prefix_workspace_bytes(case.num_seqs, case.num_q_heads,
                                                    case.num_kv_heads, case.head_dim,
                                                    case.block_size, max_ctx, kvt, part_tokens)
        g_gs, g_gpb = dev(case.group_start), dev(case.group_prefix_blocks)
        max_group = int(np.diff(case.group_start).max())
        max_prefix = max(1, int(case.group_prefix_blocks.max()))
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # longest contexts first (stable, so equal lengths keep the batch order); an identity order
    # is not passed at all
    order = np.argsort(-np.asarray(case.context_lens), kind="stable").astype(np.int32)
    use_order = args.seq_order == "longest" and not np.array_equal(order, np.arange(case.num_seqs))
    g_order = dev(order) if use_order else None
    # pa_decode_append takes one new row per sequence, at its newest position L - 1
    newest = [int(case.block_tables[b, (int(L) - 1) // case.block_size]) * case.block_size
              + (int(L) - 1) % case.block_size if int(L) > 0 else -1
              for b, L in enumerate(case.context_lens)]
    fused = (args.append == "fused" and nk.shape[0] == case.num_seqs
             and np.array_equal(np.asarray(slots, np.int64), np.asarray(newest, np.int64)))

    def decode():
        if fused and shared:
            pa.pa_decode_shared_prefix_append(out, q, g_nk, g_nv, kc, vc, g_slots, tables, lens,
                                              g_gs, g_gpb, float(case.scale),
                                              max_group_seqs=max_group,
                                              max_prefix_blocks=max_prefix, k_scale=ks,
                                              v_scale=vs, max_context_len=max_ctx,
                                              partition_tokens=part_tokens, workspace=ws,
                                              seq_order=g_order)
        elif fused:
            pa.pa_decode_append(out, q, g_nk, g_nv, kc, vc, g_slots, tables, lens,
                                float(case.scale), k_scale=ks, v_scale=vs,
                                max_context_len=max_ctx, partition_tokens=part_tokens,
                                workspace=ws, seq_order=g_order)
        elif shared:
            pa.pa_decode_shared_prefix(out, q, kc, vc, tables, lens, g_gs, g_gpb, float(case.scale),
                                       max_group_seqs=max_group,
                                       max_prefix_blocks=max_prefix, k_scale=ks, v_scale=vs,
                                       max_context_len=max_ctx, partition_tokens=part_tokens,
                                       workspace=ws, seq_order=g_order)
        else:
            pa.pa_decode(out, q, kc, vc, tables, lens, float(case.scale), k_scale=ks, v_scale=vs,
                         max_context_len=max_ctx, partition_tokens=part_tokens, workspace=ws,
                         seq_order=g_order)

    has_pairs = g_pairs.shape[0] > 0

    def step():
        if has_pairs:
            pa.pa_copy_blocks(kc, vc, g_pairs, k_scale=ks, v_scale=vs)
        if not fused:
            pa.pa_kv_write(g_nk, g_nv, kc, vc, g_slots, k_scale=ks, v_scale=vs)
        decode()

    def timed(fn, n):
        """Wall-clock and HIP-event time of n back-to-back calls (events only at the ends:
        an event between kernels adds a cache flush of its own)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n, e0.elapsed_time(e1) * 1e-3 / n

    if args.calibrate:
        progress("calibration copy: 3 x 256 MiB read + 256 MiB written")
        src = torch.ones(2 ** 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The attainable-bandwidth probe runs first: it also brings the idle GPU up to speed before
    # the warm-up steps.
    attainable = None
    if args.probe_gib > 0:
        progress(f"streaming-read probe over {args.probe_gib:g} GiB")
        buf = torch.empty(int(args.probe_gib * 2 ** 30), dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        times = []
        for i in range(12):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pa.stream_read_probe(buf, sink)
            e1.record(stream)
            e1.synchronize()
            if i >= 2:
                times.append(e0.elapsed_time(e1) * 1e-3)
        attainable = buf.numel() / statistics.median(times) / 1e9
        del buf

    progress(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Optionally the step is captured once into a HIP graph and replayed. Nothing in the step
    # allocates or clears memory (the decode counters return to zero by themselves), so replays
    # are identical to eager steps.
    graph = None
    if args.graph:
        progress("capturing the step into a HIP graph")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        ref_out = out.clone()
        step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "graph replay differs"

    progress(f"timing {args.steps} steps ({'eager' if graph is None else 'graph replay'})")
    wall_step, event_step = timed(step if graph is None else graph.replay, args.steps)
    ms_per_step = wall_step * 1e3
    eager_wall, _ = timed(step, args.steps) if graph is not None else (wall_step, None)
    progress(f"timing {args.steps} decode calls")
    _, event_call = timed(decode, args.steps)
    avg_call_ms = event_call * 1e3
    separate_ms = None
    if fused:
        # the same step with the append as its own launch (pa_kv_write, then pa_decode), for
        # comparison: bit-identical results
        def step_separate():
            if g_pairs.shape[0]:
                pa.pa_copy_blocks(kc, vc, g_pairs, k_scale=ks, v_scale=vs)
            pa.pa_kv_write(g_nk, g_nv, kc, vc, g_slots, k_scale=ks, v_scale=vs)
            if shared:
                pa.pa_decode_shared_prefix(out, q, kc, vc, tables, lens, g_gs, g_gpb,
                                           float(case.scale), max_group_seqs=max_group,
                                           max_prefix_blocks=max_prefix, k_scale=ks, v_scale=vs,
                                           max_context_len=max_ctx, partition_tokens=part_tokens,
                                           workspace=ws, seq_order=g_order)
            else:
                pa.pa_decode(out, q, kc, vc, tables, lens, float(case.scale), k_scale=ks,
                             v_scale=vs, max_context_len=max_ctx, partition_tokens=part_tokens,
                             workspace=ws, seq_order=g_order)

        # its own warm-up: the append kernel has not run in this process yet (its first
        # launch loads the code object)
        for _ in range(max(1, min(args.warmup, 20))):
            step_separate()
        progress(f"timing {args.steps} steps with the append launched separately")
        _, event_sep = timed(step_separate, args.steps)
        separate_ms = event_sep * 1e3

    # per-call timing after evicting L2 and the 256 MiB Infinity Cache with a 1 GiB read (a
    # read leaves no dirty lines behind whose write-back would slow the timed call)
    flushed = None
    if args.flushed_calls > 0:
        progress(f"timing {args.flushed_calls} flushed calls")
        fa = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda")
        fsink = torch.zeros(1, dtype=torch.int32, device="cuda")
        times = []
        for _ in range(args.flushed_calls):
            pa.stream_read_probe(fa, fsink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            decode()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        times.sort()
        flushed = {"median_us": statistics.median(times), "p10_us": times[len(times) // 10],
                   "p90_us": times[(9 * len(times)) // 10]}
        del fa

    swap = None
    if args.swap_blocks > 0:
        n = min(args.swap_blocks, case.num_blocks)
        progress(f"swap of {n} blocks to pinned host memory and back")
        hk = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype).pin_memory()
        hv = torch.empty_like(hk).pin_memory()
        hks = hvs = None
        if ks is not None:
            hks = torch.empty((n, case.num_kv_heads), dtype=torch.float32).pin_memory()
            hvs = torch.empty_like(hks).pin_memory()
        live = np.unique(np.concatenate([row[: -(-int(L) // case.block_size)]
                                         for row, L in zip(case.block_tables, case.context_lens)]))
        ids = torch.from_numpy(np.ascontiguousarray(live[:n])).int().cuda()
        n = int(ids.numel())
        out_map = torch.stack([ids, torch.arange(n, dtype=torch.int32, device="cuda")], 1).contiguous()
        in_map = torch.stack([out_map[:, 1], out_map[:, 0]], 1).contiguous()
        nbytes = 2 * n * int(np.prod(kc.shape[1:])) * kc.element_size()

        def swap_out():
            pa.pa_swap_blocks(kc, vc, hk, hv, out_map, src_k_scale=ks, src_v_scale=vs,
                              dst_k_scale=hks, dst_v_scale=hvs)

        def swap_in():
            pa.pa_swap_blocks(hk, hv, kc, vc, in_map, src_k_scale=hks, src_v_scale=hvs,
                              dst_k_scale=ks, dst_v_scale=vs)

        swap_out(); swap_in()
        t_out = timed(swap_out, 5)[1]
        t_in = timed(swap_in, 5)[1]
        swap = {"blocks": n, "bytes": nbytes, "out_gbs": nbytes / t_out / 1e9,
                "in_gbs": nbytes / t_in / 1e9, "host": "pinned (hipHostMalloc via torch)"}
        del hk, hv

    kvb = kv_bytes(case)
    seq_tokens = int(case.context_lens.sum())
    value = kvb / (ms_per_step * 1e-3) / 1e9
    call_bytes = decode_call_bytes(case)
    if fused:  # the new rows: read from k_new / v_new and written to the cache
        call_bytes += 2 * 2 * int(np.asarray(nk).nbytes)
    achieved = call_bytes / (avg_call_ms * 1e-3) / 1e9
    kfam = decode_kernel_family(case.num_q_heads // case.num_kv_heads, shared)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_source_sha256") == kernel_source_hash() and tr.get("workload") == args.workload:
            traffic = tr.get("hbm_bytes_per_call")
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": ((f"pa_decode_shared_prefix_append (prefix pass prefill_kernel<PREFIX> + "
                            f"{kfam} with the step's append fused)") if shared and fused else
                           (f"pa_decode_shared_prefix (prefix pass prefill_kernel<PREFIX> + "
                            f"{kfam}, merge fused)") if shared else
                           (f"pa_decode_append ({kfam} with the step's append and the "
                            "cross-partition merge fused)") if fused else
                           f"pa_decode ({kfam}, cross-partition merge fused)"),
                "algorithmic_bytes_per_call": call_bytes, "avg_call_us": avg_call_ms * 1e3,
                "timing": "HIP events around the timed back-to-back calls of the entry point "
                          "named in kernel"}
    quality = None
    if args.quality:
        progress("E4M3 quality report (oracle on the host, pa_decode on the GPU)")
        quality = e4m3_quality()
    line = {
        "metric": "paged decode attention: KV GB/s (% of HBM peak) + seq-tokens/s, 8B-shaped, 1 GPU",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "event_ms_per_step": event_step * 1e3,
        "launch": "eager" if graph is None else "hip graph replay of the step",
        "eager_ms_per_step": eager_wall * 1e3,
        "separate_append_event_ms_per_step": separate_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) fp16 q/K/V, scattered blocks, NaN-poisoned unused slots)",
        "config": {"workload": describe(case), "num_seqs": case.num_seqs,
                   "max_context_len": max_ctx, "q_heads": case.num_q_heads,
                   "kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "block_size": case.block_size, "kv_dtype": case.kv_dtype,
                   "step": ("copy_blocks(pairs) + decode_append (kv_write of 1 token/seq fused "
                            "into the decode launch)" if case.kv_dtype == "f16" else
                            "copy_blocks(pairs) + decode_append (E4M3 kv_write of 1 token/seq "
                            "and the decode in one call)") if fused else
                           "copy_blocks(pairs) + kv_write(1 token/seq) + decode",
                   "partition_tokens": part_tokens if part_tokens else "auto",
                   "decode": "shared_prefix" if shared else "plain",
                   "seq_order": "longest first" if use_order else "batch order",
                   "append": ("separate" if not fused else "fused" if case.kv_dtype == "f16"
                              else "in the call (E4M3: fused into the decode launch when one head "
                                   "tile covers a KV head's query heads, else the append kernel "
                                   "first)")},
        "hbm_frac": value / HBM_PEAK_GBS,
        "attainable_read_gbs": attainable,
        "frac_of_attainable": None if attainable is None else value / attainable,
        "seq_tokens_per_s": seq_tokens / (ms_per_step * 1e-3),
        "kv_bytes_per_step": kvb,
        "flushed_decode": flushed,
        "swap": swap,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "e4m3_quality": quality,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

/*
 * pa.h — paged decode attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The KV cache is a pool of fixed-size blocks that need not be contiguous in memory; each
 * sequence keeps a block table whose entry i names the physical block that holds its logical
 * block i, and attention reads the scattered blocks through that table
 * ("serving-paged-attention", section "블록으로 쪼개고 표로 잇는다"; the talk summary's vLLM
 * paragraph: logically contiguous, physically scattered). New tokens are placed by slot
 * ("vLLM의 핵심 이해: PagedAttention", section 6, TokenTable / SlotAllocator), and a shared
 * block that is still filling is copied before a sequence writes into it
 * ("serving-paged-attention", section "공유는 표를 베끼는 일이 된다").
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked otherwise; every call only enqueues work on
 *     `stream` (a hipStream_t; NULL = the legacy default stream) and returns without waiting.
 *   - The caller owns every buffer (including the decode workspace). The library allocates,
 *     frees and synchronises nothing and keeps no per-call state; calls are re-entrant. The one
 *     exception is pa_decode_append_noalloc, whose workspace is a fixed device array inside
 *     the library (one per GPU, shared by every such call on that GPU).
 *   - Only host-side scalars and pointers are validated, before anything is enqueued. On a
 *     validation failure nothing is enqueued and the status code says why. Launch failures
 *     return PA_ERR_HIP; pa_last_hip_error() then gives the hipError_t (per calling thread).
 *   - Device-side data is NOT validated (documented preconditions below); violating them gives
 *     wrong values, but out-of-range block ids and slots are clamped or skipped on the device,
 *     so no access leaves the caller's buffers.
 *   - All arrays are row-major and densely packed.
 *
 * Layouts (S sequences, Hq query heads, Hkv KV heads, D head dim, BS block size, NB blocks):
 *   q, out        [S, Hq, D]            fp16
 *   k_cache       [NB, Hkv, BS, D]      fp16, or uint8 OCP FP8 E4M3 codes
 *   v_cache       [NB, Hkv, BS, D]      same type as k_cache
 *   k_scale       [NB, Hkv]             fp32 per (block, KV head) dequant scale (E4M3 only)
 *   v_scale       [NB, Hkv]             fp32
 *   block_tables  [S, max_blocks_per_seq] int32 physical block ids
 *   context_lens  [S]                   int32 tokens attended per sequence
 *   k, v (new)    [T, Hkv, D]           fp16
 *   slot_mapping  [T]                   int64, slot = block * BS + offset, < 0 = skip
 *   block_mapping [P, 2]                int32 (src, dst) pairs
 * Supported: D in {64, 128}; BS in {8, 16, 32, 64}; any Hq that is a multiple of Hkv.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 2

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, Hq % Hkv != 0, ...     */
  PA_ERR_UNSUPPORTED = 2, /* head_dim / block_size / dtype combination not compiled in     */
  PA_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than required             */
  PA_ERR_HIP = 4          /* a HIP launch failed; see pa_last_hip_error()                  */
} pa_status;

typedef enum {
  PA_KV_F16 = 0,      /* IEEE binary16 keys and values                                      */
  PA_KV_FP8_E4M3 = 1  /* OCP FP8 E4M3 codes (bias 7, max 448, S.1111.111 = NaN), with one     */
                      /* fp32 scale per (block, KV head): value = decode(code) * scale        */
} pa_kv_dtype;

/* Returns PA_ABI_VERSION of the loaded library. */
int pa_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* pa_status_str(int status);

/* hipError_t value behind the most recent PA_ERR_HIP returned on the calling thread (0 if none). */
int pa_last_hip_error(void);

/*
 * Split-context partition size pa_decode uses for this shape: context tokens handled by one
 * workgroup. partition_tokens = 0 asks for the automatic choice: one partition per sequence
 * (the smallest power of two >= max_context_len, at most 4096 and valid for the block size)
 * when that grid still has at least 512 workgroups (two per compute unit of a 256-CU gfx950;
 * 256 when G = Hq / Hkv >= 4, which runs on matrix-core tiles); otherwise the largest power of
 * two in [256, 4096], at most max_context_len / 2, that still gives at least 1024 workgroups
 * (256 when G >= 4), else 256. Workgroups = num_seqs x Hkv x head tiles per KV head x partitions.
 * (pa_decode_shared_prefix keeps G = 4 on the vector-ALU kernel and applies these rules with
 * G >= 5 in place of G >= 4; pa_decode_shared_prefix_workspace_bytes resolves 0 that way.)
 * An explicit value must be a power of two in [256, 4096] with value <= 256 * block_size.
 * Returns 0 if the arguments are invalid.
 */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                   int32_t kv_dtype, int32_t partition_tokens);

/* Bytes of device workspace pa_decode needs for these arguments (same meaning as in pa_decode;
 * max_context_len must be the value pa_decode will see, > 0); 0 if none is needed (every
 * sequence fits one partition) or if the arguments are invalid. The value is a multiple of
 * 16384. A larger workspace serves every call whose own size fits in it (see below).
 *
 * Workspace layout. The split partitions of a sequence are merged by the workgroup that
 * arrives last, which needs one arrival counter per (sequence, head group) besides the partial
 * results themselves (talk summary, FlashAttention paragraph: partial softmax states combine
 * exactly). A workspace of W bytes (the workspace_bytes argument) is split by W alone: the first
 * Z = 256 * floor(W / 16384) bytes are the counter zone, the rest the partial zone. Every call
 * keeps its counters at the start of the counter zone and its partials at the start of the
 * partial zone, so calls of different shapes (more sequences, more head groups, other partition
 * sizes) can share one buffer: no call reads as a counter a byte that another call wrote as a
 * partial. Rules:
 *   - pass the same workspace_bytes in every call on one buffer (the zones depend on it);
 *   - the counter zone must be zero before the first call: zero-fill the buffer, or call
 *     pa_decode_workspace_reset. Every call that runs to completion leaves it zero again;
 *   - calls sharing a workspace must not overlap in time (same stream, or synchronised);
 *   - if a call did not run to completion (an aborted or failed stream) or calls did overlap,
 *     counters may be left non-zero, and a later call would then leave some outputs unwritten:
 *     call pa_decode_workspace_reset before the next use. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t kv_dtype, int32_t partition_tokens);

/*
 * pa_decode_workspace_reset — enqueue a clear of a decode workspace's counter zone (its first
 * 256 * floor(workspace_bytes / 16384) bytes) on `stream`, as a kernel (graph-capturable, no
 * memset node). Use it on fresh memory instead of a full zero-fill, and to recover after a call
 * that did not complete or calls that overlapped (see the workspace layout above). The partial
 * zone needs no clearing. A workspace smaller than 16384 bytes has no counter zone: PA_OK, nothing
 * enqueued.
 * Validated: workspace non-NULL and 256-byte aligned when there is something to clear.
 */
int pa_decode_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode — one query token per sequence attends over its paged KV cache.
 *
 * For every sequence b with L = context_lens[b] and every query head h, with G = Hq / Hkv and
 * g = h / G (query heads share KV heads in contiguous groups: MHA G = 1, GQA, MQA Hkv = 1; the
 * talk summary's attention-heads paragraph):
 *     K_b[t] = k_cache[block_tables[b, t / BS], g, t % BS, :]   (t < L, likewise V_b)
 *     out[b, h, :] = softmax(scale * K_b q[b, h]) V_b           (fp32 accumulate, fp16 out)
 * evaluated with an online softmax (running max, running sum, running output) over tiles and
 * split across context partitions of partition_tokens tokens that are merged exactly (talk
 * summary, FlashAttention paragraph). A sequence that fits one partition is finished by its
 * workgroup; split sequences are merged by a second small kernel on `stream` (groups of at most
 * three query heads per KV head, the vector-ALU kernel, in batch order) or by the workgroup
 * that finishes a sequence's last partition (larger groups, the matrix-core kernel, and any
 * call with seq_order). L = 0 gives out = 0. For E4M3 caches each value is
 * decode(code) * scale[block, g] before use. context_lens counts every token to attend,
 * including one appended by this step's pa_kv_write.
 *
 *   seq_order        NULL, or [num_seqs] int32 device array, a permutation of 0 .. num_seqs-1:
 *                    the order in which sequences are dispatched (grid row y decodes sequence
 *                    seq_order[y]); out stays in batch order. With uneven lengths, putting the
 *                    longest contexts first lets their partitions start first instead of forming
 *                    the tail of the grid ("serving-paged-attention", section "블록 크기는 어떻게
 *                    정하나": requests of very different lengths share one batch); with an order
 *                    given, the vector-ALU kernel also dispatches the last partitions of the
 *                    split contexts first, so the grid ends with the shortest pieces. Results are
 *                    bit-identical for any order. An entry outside [0, num_seqs) is clamped; a
 *                    non-permutation gives wrong outputs (and may leave counters that
 *                    pa_decode_workspace_reset clears), never an access outside the buffers.
 *   max_context_len  host-side upper bound on context_lens[] used to size the grid;
 *                    <= 0 means max_blocks_per_seq * block_size.
 *   partition_tokens 0 = automatic, else an explicit split size (see
 *                    pa_decode_partition_tokens). Results are bit-identical for a given
 *                    partition size; different sizes round differently (within tolerance).
 *   scale            softmax scale (finite), usually 1/sqrt(head_dim).
 *   workspace        device memory, 256-byte aligned, of workspace_bytes >=
 *                    pa_decode_workspace_bytes(...) bytes (may be NULL when that size is 0),
 *                    under the rules of the workspace layout above: its counter zone is zero
 *                    before the first call (zero-fill, or pa_decode_workspace_reset), every
 *                    completed call leaves it zero, and one buffer, always passed with the
 *                    same workspace_bytes, serves later calls of any shape that fit in it.
 *                    Calls that share a workspace must not overlap in time.
 *   num_blocks       NB, the number of blocks in each cache.
 * Preconditions (not checked): 0 <= context_lens[b] <= max_context_len (as passed or implied);
 * 0 <= block_tables[b, i] < num_blocks for i < ceil(L / BS) (later entries are never read);
 * out does not alias any input. Violations give wrong values
 * but no access outside the buffers: block ids are clamped into [0, num_blocks), tokens beyond
 * the grid's partitions are dropped.
 * Validated: non-NULL pointers (k_scale/v_scale must be NULL for fp16 and non-NULL for E4M3),
 * 16-byte alignment of q, out, k_cache, v_cache; 4-byte alignment of the int arrays (seq_order
 * included) and scales;
 * positive sizes; Hq % Hkv == 0; supported head_dim, block_size and dtype; partition_tokens
 * (PA_ERR_UNSUPPORTED if it is not a valid explicit size); workspace size and alignment.
 * Deterministic: results depend only on logical token positions, not on physical ids.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_tables,
              const int32_t* context_lens,
              const int32_t* seq_order, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
              int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_tokens,
              float scale, int32_t kv_dtype, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * pa_decode_append — one decode step's append and attention in one call: the new token of
 * every sequence is stored into the paged cache at its slot and attended together with the
 * tokens already cached.
 *
 * A decode step writes the new token's key and value to the slot the block table gives it
 * ("vLLM의 핵심 이해: PagedAttention", section 6: a token maps to a page and a position in it)
 * and then attends over all tokens so far, the new one included ("serving-paged-attention",
 * section "캐시가 얼마나 큰지부터"). This call computes exactly
 *     pa_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens = num_seqs, ...);
 *     pa_decode(out, q, k_cache, v_cache, ...);
 * with bit-identical out, caches and scales. For fp16 caches it is one kernel launch: every
 * workgroup covering position context_lens[b] - 1 takes that token's K/V from k_new/v_new[b]
 * instead of the cache, and one workgroup per (sequence, KV head) stores them at
 * slot_mapping[b]. E4M3 caches (whose append may rescale the block) are one launch too when one
 * head tile covers all query heads of a KV head (1 to 3 query heads per KV head on the vector
 * ALU; 4 to 32 in one matrix-core tile): the workgroup that reads the sequence's last block
 * applies the block-scale policy of pa_kv_write itself (the rows encoded under the updated
 * scale, the block's earlier codes re-encoded in registers when the scale grows) and stores
 * codes and scales. Other E4M3 head layouts (several workgroups per KV head) launch the append
 * kernel and then the decode kernel, both on `stream`.
 *
 *   k_new, v_new   [num_seqs, Hkv, D] fp16, device, 16-byte aligned: row b is sequence b's new
 *                  token (one token per sequence, in sequence order).
 *   slot_mapping   [num_seqs] int64, device, 8-byte aligned: block * block_size + offset of that
 *                  token; < 0 (or >= num_blocks * block_size) = sequence b appends nothing this
 *                  step and its cache is attended as it is.
 *   k_scale, v_scale  as for pa_decode; for E4M3 caches they are updated by the append.
 * Other arguments as for pa_decode (same workspace size: pa_decode_workspace_bytes).
 * Precondition (not checked), beyond pa_decode's: a non-negative slot_mapping[b] is the slot of
 * position context_lens[b] - 1 in b's table (the single-call fusion relies on it) and slots are
 * unique. Violations give wrong values, never an access outside the buffers.
 * Validated: as pa_decode, plus non-NULL k_new, v_new, slot_mapping with the alignments above,
 * num_blocks * block_size < 2^31 and num_seqs * Hkv * D / 8 < 2^31.
 */
int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                     const int64_t* slot_mapping, const int32_t* block_tables,
                     const int32_t* context_lens,
              const int32_t* seq_order, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                     int32_t partition_tokens, float scale, int32_t kv_dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Size of the library's own decode workspace (per GPU) used by pa_decode_append_noalloc. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * pa_decode_append_noalloc — pa_decode_append without a caller-provided workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It allocates nothing and calls no allocating routine.
 *
 * Arguments, semantics and results are those of pa_decode_append (bit-identical outputs and
 * caches for the same arguments), minus workspace and workspace_bytes: the split-context
 * partials and arrival counters live in a file-scope device array of PA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that each GPU the library runs on holds until the process ends.
 *   - A call whose pa_decode_workspace_bytes(...) exceeds PA_NOALLOC_SCRATCH_BYTES returns
 *     PA_ERR_WORKSPACE before anything is enqueued (choose a larger partition_tokens, or use
 *     pa_decode_append with a workspace).
 *   - The first call on a GPU that needs the array looks up its device address (the current
 *     device's copy, hipGetSymbolAddress) and enqueues a clear of its counters on `stream`; that
 *     first call should not be under graph capture. Later calls reuse the address.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents; each
 *     completed call leaves its counters at zero. Calls that overlap in time on one GPU (other
 *     streams, other threads) race on the array and give wrong results: serialise them.
 * The current device (hipGetDevice) must be the device of the buffers and of `stream`.
 * Validated: as pa_decode_append; PA_ERR_WORKSPACE as above; PA_ERR_UNSUPPORTED for a device
 * ordinal >= 64.
 */
int pa_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             const int64_t* slot_mapping, const int32_t* block_tables,
                             const int32_t* context_lens,
              const int32_t* seq_order, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, int32_t partition_tokens, float scale,
                             int32_t kv_dtype, void* stream);

/*
 * pa_decode_shared_prefix — pa_decode for batches in which groups of sequences share leading
 * blocks (one system prompt behind many requests, or the siblings of parallel sampling), with
 * the shared blocks read once per KV head for the whole group.
 *
 * Sharing a prefix makes block tables point at the same physical blocks ("serving-paged-
 * attention", section "공유는 표를 베끼는 일이 된다": 100 requests behind one 512-token system
 * prompt). Plain decode still reads those blocks once per sequence. Here the call runs in two
 * passes on `stream`:
 *   1. prefix pass: for each group g (sequences group_start[g] .. group_start[g+1]-1) and KV
 *      head, the first group_prefix_blocks[g] blocks of the group's first member's table are
 *      attended by the G query rows of every member at once, as matrix-core products, giving
 *      each (member, query head) unnormalised partials (running max, running sum, weighted
 *      value sum), one per slice of the prefix tokens;
 *   2. decode pass: each sequence's remaining tokens [prefix, L) are attended exactly as in
 *      pa_decode, and the workgroup that finishes a sequence merges the prefix partial with the
 *      partition partials, exactly (talk summary, FlashAttention paragraph: partial softmax
 *      states combine without approximation).
 * The output is out[b, h, :] of pa_decode for the same inputs, up to rounding (the prefix
 * products round the probabilities to fp16 before the product with V).
 *
 *   group_start          [num_groups + 1] int32, device: increasing sequence indices from 0 to
 *                        num_seqs; a sequence that shares nothing is a group of its own (or
 *                        has group_prefix_blocks 0).
 *   group_prefix_blocks  [num_groups] int32, device: full blocks shared by every member of the
 *                        group, taken from the first member's table (0 = none).
 *   max_group_seqs       host bound on every group's size (sizes the prefix pass's grid).
 *   max_prefix_blocks    host bound on group_prefix_blocks[] (>= 1). The prefix pass covers at
 *                        most min(max_prefix_blocks, max_blocks_per_seq, 4096,
 *                        max_context_len / block_size) blocks of a group; shared blocks beyond
 *                        that are attended per sequence, which gives the same result. The
 *                        prefix is cut into at most 4 slices of at least 128 tokens, one
 *                        workgroup each, so that short prefixes still spread over the GPU.
 *   workspace            >= pa_decode_shared_prefix_workspace_bytes(...) bytes, under the
 *                        rules of pa_decode's workspace (always needed here).
 * Other arguments as for pa_decode.
 * Preconditions (not checked), beyond pa_decode's: every member's first group_prefix_blocks[g]
 * table entries equal the first member's, and group_prefix_blocks[g] * block_size <= the
 * member's context length. Violations give wrong values, never an access outside the buffers.
 * Validated: as pa_decode, plus non-NULL 4-byte aligned group arrays, num_groups >= 1,
 * 1 <= max_group_seqs <= num_seqs, max_prefix_blocks >= 1, and the prefix pass's grid
 * (ceil(max_group_seqs * G / 128) * Hkv * num_groups * slices workgroups) < 2^31.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t max_context_len,
                                               int32_t kv_dtype, int32_t partition_tokens);
int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, const int32_t* context_lens,
              const int32_t* seq_order,
                            const int32_t* group_start, const int32_t* group_prefix_blocks,
                            int32_t num_groups, int32_t max_group_seqs,
                            int32_t max_prefix_blocks, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, int32_t partition_tokens, float scale,
                            int32_t kv_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * pa_decode_shared_prefix_append — one decode step for batches with shared prefixes: the new
 * token of every sequence is stored into the paged cache at its slot and the batch is decoded
 * as by pa_decode_shared_prefix, in one call. It computes exactly
 *     pa_kv_write(k_new, v_new, ..., slot_mapping, num_tokens = num_seqs, ...);
 *     pa_decode_shared_prefix(out, q, ...);
 * with bit-identical out and caches: a step of 100 requests behind one system prompt appends
 * one token to each private tail and attends over the shared prompt and the tail
 * ("serving-paged-attention", section "공유는 표를 베끼는 일이 된다"). For fp16 caches the decode
 * launch stores and attends the new rows itself (as pa_decode_append); for E4M3 caches the
 * append kernel runs first.
 * Arguments: those of pa_decode_append (k_new, v_new, slot_mapping, writable scales) and of
 * pa_decode_shared_prefix (group_start, group_prefix_blocks, num_groups, max_group_seqs,
 * max_prefix_blocks; same workspace size: pa_decode_shared_prefix_workspace_bytes).
 * Precondition (not checked), beyond those two: an appending sequence's new position
 * context_lens[b] - 1 lies after its group's shared blocks (group_prefix_blocks[g] *
 * block_size <= context_lens[b] - 1): a token is never written into a shared block (copy it
 * first, pa_copy_blocks). Violations give wrong values, never an access outside the buffers.
 * Validated: as pa_decode_append and pa_decode_shared_prefix.
 */
int pa_decode_shared_prefix_append(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    float* k_scale, float* v_scale, const int64_t* slot_mapping, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* seq_order, const int32_t* group_start,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t max_group_seqs,
    int32_t max_prefix_blocks, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t partition_tokens, float scale, int32_t kv_dtype,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill — causal attention of a chunk of new tokens per sequence over its paged KV cache
 * (prefill, or one chunk of a chunked prefill).
 *
 * Prefill turns the prompt into KV-cache entries with large matrix products and is bound by
 * arithmetic, while decode is bound by reading the cache ("LLM 추론 확장, 품질·비용 절충 필수",
 * prefill and decode paragraphs). The chunk's keys and values are appended first (pa_kv_write);
 * then, for sequence b with n = query_start[b+1] - query_start[b] query rows and
 * L = context_lens[b] tokens in the cache (the chunk being the last n of them), every query
 * head h (KV head g = h / G) and chunk token j < n at position p = L - n + j:
 *     out[query_start[b] + j, h, :] = softmax(scale * K_b[0..p] q[query_start[b] + j, h])
 *                                     V_b[0..p]
 * with K_b, V_b read through the block table as in pa_decode (fp32 accumulation, fp16 out;
 * E4M3 values are decode(code) * scale[block, g]). Scores and probabilities go through fp16
 * matrix-core products, the probabilities rounded to fp16 before the product with V.
 * A decode step is the case n = 1.
 *
 *   q, out           [num_tokens, Hq, D] fp16, the chunks of all sequences back to back.
 *   query_start      [num_seqs + 1] int32 device array: first row of each sequence's chunk
 *                    in q / out, then num_tokens.
 *   max_query_len    host-side upper bound on every n (sizes the grid).
 *   max_context_len  host-side upper bound on context_lens[]; at most max_blocks_per_seq *
 *                    block_size and at most 4096 * block_size (the kernel keeps a sequence's
 *                    block ids on chip).
 * Preconditions (not checked): query_start non-decreasing from 0 to num_tokens;
 * n <= max_query_len; n <= context_lens[b] <= max_context_len; block ids of the first
 * ceil(L / BS) table entries in [0, num_blocks); out does not alias any input. Violations give
 * wrong values but no access outside the buffers: row ranges are clamped into [0, num_tokens),
 * n to max_query_len, L to max_context_len, block ids into [0, num_blocks); rows at a position
 * below 0 are written as zeros.
 * Validated: non-NULL pointers (scales as in pa_decode), 16-byte alignment of q, out and the
 * caches; 4-byte alignment of the int arrays; sizes; Hq % Hkv == 0; supported head_dim,
 * block_size and dtype; the grid (max_query_len * G / 128 * Hkv * num_seqs workgroups) < 2^31.
 * num_tokens == 0 returns PA_OK without launching. Needs no workspace; deterministic.
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const float* k_scale, const float* v_scale, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
               int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
               int32_t max_query_len, int32_t max_context_len, float scale, int32_t kv_dtype,
               void* stream);

/*
 * pa_kv_write — slot-mapped append of new keys and values.
 *
 * For each token t < num_tokens with slot = slot_mapping[t] >= 0, writes
 *     k_cache[slot / BS, h, slot % BS, :] = k[t, h, :]   and the same for v, for all h.
 * Tokens with a negative slot, or a slot >= num_blocks * block_size, are skipped. Nothing else
 * in the caches changes (except, for E4M3, the earlier codes of a block whose scale grows).
 *
 * PA_KV_FP8_E4M3 caches (k_scale, v_scale non-NULL) are written under this scale policy, per
 * (token, KV head), all in fp32 with IEEE division:
 *     s_prev = scale[blk, h], or 0 when the token lands at offset 0 (the block starts fresh);
 *     a = max |x| over the token's row; s = a / 448 if a > s_prev * 448, else s = s_prev;
 *     s = 1 if it is still 0; when s grows and the block already holds tokens, each earlier
 *     code c of that (block, head) becomes enc((dec(c) * s_prev) / s); the token is stored as
 *     enc(x / s) and scale[blk, h] = s. enc clamps to [-448, 448] and rounds to nearest even.
 * The scale thus stays >= the block's max |value| / 448, the rule used to quantize whole blocks.
 *
 * For E4M3 caches, consecutive tokens of the call that land in the same block (a run, e.g. a
 * prefill chunk's tokens in order) are applied in that order, each under the policy above.
 * Precondition (not checked): non-negative slots are distinct; for E4M3 caches the tokens that
 * land in one block are consecutive in the call.
 * Validated: pointers (scales NULL for fp16, non-NULL for E4M3), 16-byte alignment of k, v,
 * caches; 8-byte alignment of slot_mapping; sizes; num_blocks * block_size < 2^31.
 */
int pa_kv_write(const void* k, const void* v, void* k_cache, void* v_cache, float* k_scale,
                float* v_scale, const int64_t* slot_mapping, int32_t num_tokens,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t kv_dtype, void* stream);

/*
 * pa_copy_blocks — copy-on-write block copies.
 *
 * For each pair p < num_pairs: cache[dst] = cache[src] for K and V over all KV heads, and for
 * E4M3 caches also k_scale[dst, :] = k_scale[src, :] and v_scale[dst, :] = v_scale[src, :],
 * with (src, dst) = block_mapping[p]. Every copy reads the state before the call.
 * Pairs with an id outside [0, num_blocks) are skipped. Precondition (not checked):
 * destinations are distinct and none is a source. Validated: pointers (scales NULL for fp16, non-NULL for E4M3), 16-byte alignment
 * of the caches, sizes, num_blocks * block_size < 2^31.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int32_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                   void* stream);

/*
 * pa_swap_blocks — move whole blocks between two pools, e.g. out of the device pool into a
 * pinned host pool and back (preemption by swap: "serving-paged-attention", section
 * "그래도 넘칠 때 — 선점": a request's blocks go to CPU memory and return later, trading PCIe
 * time for the recomputation).
 *
 * For each pair p with (src, dst) = block_mapping[p]: dst_k[dst] = src_k[src] and
 * dst_v[dst] = src_v[src] over all KV heads (a block is Hkv*BS*D elements), and for E4M3 pools
 * dst_*_scale[dst, :] = src_*_scale[src, :]. src ids index the source pool (src_num_blocks
 * blocks), dst ids the destination pool (dst_num_blocks blocks); pairs with an id out of range
 * are skipped. Either pool may be device memory or pinned host memory allocated with
 * hipHostMalloc (reachable from the device through its host pointer); block_mapping is device
 * memory. Both pools share Hkv, BS, D and dtype.
 * Precondition (not checked): destinations are distinct and, when both pools are the same
 * buffer, disjoint from the sources.
 * Validated: pointers (all four scale pointers NULL for fp16, non-NULL for E4M3), 16-byte
 * alignment of the pools, sizes, num_kv_heads <= 256.
 */
int pa_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scale,
                   const float* src_v_scale, void* dst_k, void* dst_v, float* dst_k_scale,
                   float* dst_v_scale, const int32_t* block_mapping, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t src_num_blocks, int32_t dst_num_blocks, int32_t kv_dtype,
                   void* stream);

/*
 * pa_stream_read_probe — measurement utility, not part of the decode path.
 *
 * Reads the first floor(bytes / 16) * 16 bytes of `buf` once with 16-byte loads spread over
 * the whole GPU, so that timing it gives the attainable HBM read bandwidth that pa_decode's
 * KV bandwidth is compared against. `sink` (4 bytes) is written only in the rare case that
 * the folded data equals a fixed constant; its contents are meaningless.
 * Validated: non-NULL, bytes >= 16, buf 16-byte aligned, sink 4-byte aligned.
 */
int pa_stream_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

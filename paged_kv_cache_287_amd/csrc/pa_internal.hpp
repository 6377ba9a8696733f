// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// ---- decode geometry -------------------------------------------------------------------
// A workgroup of kWaves wavefronts owns one (sequence, KV-head group, context partition) and
// processes `part_tokens` consecutive logical tokens; each wave owns a quarter of them and walks
// them in tiles of kTileTokens (four 16-lane rows x four steps of one token per row). The block
// ids of a wave's tokens are held one per lane, so a wave may span at most kWave blocks:
// part_tokens / kWaves <= kWave * block_size.
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kRows = 4;
constexpr int kSteps = 4;
constexpr int kTileTokens = kRows * kSteps;
constexpr int kMinPartTokens = 256;
constexpr int kMaxPartTokens = 4096;
// Compute units of an MI355X / MI350X (gfx950): the automatic partition choice aims to give the
// grid enough workgroups to fill them.
constexpr int kNumCUs = 256;
// Accelerator complex dies of an MI355X: consecutive workgroup ids are dealt round-robin over
// them, and each has its own L2.
constexpr int kNumXcds = 8;

inline bool valid_part_tokens(int pt, int block_size) {
  if (pt < kMinPartTokens || pt > kMaxPartTokens || (pt & (pt - 1)) != 0) return false;
  return pt / kWaves <= kWave * block_size;
}

// Query heads per workgroup. Groups of 4 or more query heads per KV head (5 or more in
// shared-prefix decode, `prefix`) use the matrix-core kernel: 32 or 16 heads per tile when G is
// a multiple of 16; otherwise the group is cut into the fewest tiles of at most 32 rows that
// divide it evenly (one tile up to G = 32), padded to 16 or 32 rows. A padded tile beats the
// VALU kernel there (GQA-8 at 64 x 2,048 tokens: 51 against 76 us for fp16 KV, 45 against 64 us
// for E4M3; GQA-4, 16 rows for 4 heads: 8B shape 161.5 against 165.5-168 us per call, 64 x 2,048
// tokens with E4M3 47.5 against 57-63 us), and the VALU alternative for 5, 6 or 7 heads would
// read each K/V tile once per small head tile. Groups of 1 to 3 heads (and odd groups above 32)
// use the VALU kernel with the largest compiled tile dividing G: 8, 4, 3, 2 or 1 query heads for
// fp16 caches, at most 4 for E4M3 ones (their lanes hold 16 elements of a token, and 8 heads of
// partial outputs no longer fit the register file); at G = 2 the padded tile measured no faster.
// Shared-prefix decode keeps G = 4 on the VALU kernel, whose launch also runs the prefix pass
// (the matrix-core decode takes the prefix pass as a launch of its own: 48.6 against 42.4 us
// for the shared-prefix step of 100 sequences).
inline int mfma_rows(int group, bool prefix) {
  if (group < (prefix ? 5 : 4)) return 0;
  if (group % 32 == 0) return 32;
  if (group % 16 == 0) return 16;
  const int tiles = (group + 31) / 32;
  return group % tiles == 0 ? group / tiles : 0;
}
inline bool decode_uses_mfma(int group, bool prefix) { return mfma_rows(group, prefix) > 0; }
inline int decode_rows(int group, bool kv8, bool prefix) {
  if (decode_uses_mfma(group, prefix)) return mfma_rows(group, prefix);
  for (int gt : {8, 4, 3, 2, 1})
    if (group % gt == 0 && !(kv8 && gt > 4)) return gt;
  return 1;
}

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Automatic split-context partition size.
// (1) One partition per sequence when the smallest power of two in [256, 4096] covering the
//     longest context is valid for the block size and the grid still has `single_units`
//     workgroups (two per CU for the VALU kernel, one per CU for the matrix-core kernel): no
//     partials, no merge, and one start-up per (sequence, head group). Measured faster on every
//     uniform-length shape (8B shape 186 -> 179 us, GQA-4 64 x 2048 96 -> 89 us, MHA 335 -> 322
//     us) and on the shared-prefix workloads (equal, or 125 -> 115 us with forks).
// (2) Otherwise the largest power of two in [256, 4096], and at most half the longest context,
//     whose grid still has at least `target_units` workgroups; if none has, the smallest.
//     Longer partitions amortise each workgroup's start-up (q, table and first-tile latency) and
//     its merge; shorter ones give more parallelism and a shorter tail when lengths are uneven,
//     and splitting the longest sequences at least in two keeps one workgroup from holding a
//     whole long sequence while the rest of the GPU idles. The target is four workgroups per CU
//     for the VALU kernel and one for the matrix-core kernel, whose 16- or 32-row workgroups
//     are heavier and whose merges cost more per partition (measured best on MI355X).
inline long long decode_target_units(int group, bool prefix) {
  return decode_uses_mfma(group, prefix) ? (long long)kNumCUs : 4LL * kNumCUs;
}
inline long long decode_single_units(int group, bool prefix) {
  return decode_uses_mfma(group, prefix) ? (long long)kNumCUs : 2LL * kNumCUs;
}
inline int auto_part_tokens(int num_seqs, int units_per_seq, int max_context_len, int block_size,
                            long long target_units, long long single_units) {
  int whole = kMinPartTokens;
  while (whole < max_context_len && whole < kMaxPartTokens) whole *= 2;
  if (whole >= max_context_len && valid_part_tokens(whole, block_size) &&
      (long long)num_seqs * units_per_seq >= single_units)
    return whole;
  for (int pt = kMaxPartTokens; pt > kMinPartTokens; pt /= 2) {
    if (!valid_part_tokens(pt, block_size) || 2LL * pt > max_context_len) continue;
    const long long units = (long long)num_seqs * units_per_seq * ceil_div(max_context_len, pt);
    if (units >= target_units) return pt;
  }
  return kMinPartTokens;
}

// Workspace layout. A workspace of W bytes is split by its size alone into a counter zone
// [0, Z(W)) and a partial zone [Z(W), W), with Z(W) = 256 * floor(W / 16384): 1/64 of the
// buffer. A call keeps its arrival counters ([S * HG_total] int32) at the start of the counter
// zone and its partials ([ml: S*Hq*P*2 f32][acc: S*Hq*P*D f32], 256-byte aligned) at the start
// of the partial zone. Calls of any shape that pass the same W therefore never read a byte as a
// counter that another call wrote as a partial: the zones do not depend on the call's shape.
// Needed only when a sequence may span more than one partition (or take prefix partials).
constexpr size_t kWsGranule = 16384;
constexpr size_t kWsCounterPerGranule = 256;
inline size_t ws_counter_zone(size_t w) { return w / kWsGranule * kWsCounterPerGranule; }

struct WorkspaceLayout {
  size_t counter_bytes;  // bytes of counters this call uses (0: no workspace needed)
  size_t partial_bytes;  // bytes of partials this call uses
  size_t ml_rel, acc_rel;  // offsets of the two partial arrays inside the partial zone
  size_t total;          // smallest W whose zones hold both (a multiple of kWsGranule)
};
inline WorkspaceLayout workspace_layout(int num_seqs, int num_q_heads, int head_groups_total,
                                        int head_dim, int max_parts) {
  WorkspaceLayout w{0, 0, 0, 0, 0};
  if (max_parts <= 1) return w;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)num_seqs * num_q_heads * max_parts;
  w.counter_bytes = (size_t)num_seqs * head_groups_total * sizeof(int32_t);
  w.ml_rel = 0;
  w.acc_rel = up(rows * 2 * sizeof(float));
  w.partial_bytes = w.acc_rel + rows * head_dim * sizeof(float);
  const size_t n_ctr = (w.counter_bytes + kWsCounterPerGranule - 1) / kWsCounterPerGranule;
  const size_t per_granule = kWsGranule - kWsCounterPerGranule;
  const size_t n_par = (w.partial_bytes + per_granule - 1) / per_granule;
  w.total = (n_ctr > n_par ? n_ctr : n_par) * kWsGranule;
  return w;
}
// True when a workspace of `given` bytes holds this call's counters and partials.
inline bool workspace_fits(const WorkspaceLayout& w, size_t given) {
  const size_t z = ws_counter_zone(given);
  return w.counter_bytes <= z && w.partial_bytes <= given - z;
}

struct DecodeParams {
  _Float16* out;
  const _Float16* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // [S] grid row y decodes sequence seq_order[y] (a permutation: the caller may put the longest
  // contexts first, so that their workgroups start first); null = natural order
  const int32_t* seq_order;
  int32_t* counters;  // [S, HG_total] arrival counters; zero before and after every call
  float* ws_ml;       // [S, Hq, part_slots, 2] (running max in log2 units, running sum)
  float* ws_acc;      // [S, Hq, part_slots, D] unnormalised weighted value sums
  // Shared-prefix groups (null for plain decode): sequences [group_start[g], group_start[g+1])
  // share their first group_prefix_blocks[g] table entries, whose partial state the prefix
  // pass has already stored in slot 0; the partitions then cover the rest of each context.
  const int32_t* group_start;
  const int32_t* group_prefix_blocks;
  int32_t num_groups;
  int32_t max_prefix_blocks;  // clamp on group_prefix_blocks (<= table width, kPrefillMaxBlocks)
  int32_t prefix_split;       // prefix tokens per prefix-pass slice (multiple of 64)
  int32_t part_slots;  // partial slots per (sequence, query head): max_parts (+ kMaxPrefixSlices)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t max_parts;
  int32_t part_tokens;  // tokens per workgroup (power of two, 256..4096)
  int32_t group;        // G = Hq / Hkv
  int32_t head_groups;  // G / GT workgroups per KV head
  float scale_log2;     // softmax scale * log2(e)
  // 1: partitions only store their partials (plain stores, no arrival counter) and a second
  // kernel (launch_decode_merge) merges them; 0: the last workgroup to arrive merges in-kernel;
  // 2: as 1, and sequences with prefix partials publish theirs too (the prefix pass runs in the
  // same launch, so nothing may read its partials before the merge kernel)
  int32_t deferred_merge;
  int32_t kv_cached;  // matrix-core decode: cacheable (1) or non-temporal (0) K/V loads
  // Fused append (pa_decode_append): the new token of sequence b sits at position
  // context_lens[b] - 1; its rows k_new/v_new[b] ([S, Hkv, D] fp16) are attended in place of
  // the cache's and stored at slot_mapping[b] (< 0: no append). Null for plain decode. With an
  // E4M3 cache the rows are encoded under the block's updated scale, and when that scale grows
  // the block's earlier codes are re-encoded as they are read and stored back.
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int64_t* slot_mapping;
  uint8_t* k_cache_w;   // writable views of k_cache / v_cache for that store
  uint8_t* v_cache_w;
  float* k_scale_w;     // writable views of k_scale / v_scale (E4M3 caches)
  float* v_scale_w;
};

// ---- prefill geometry ------------------------------------------------------------------
// A prefill workgroup owns kPrefillRows query rows (chunk token x query head of one KV head) and
// holds the block ids of its attended range in LDS, so a sequence may span at most
// kPrefillMaxBlocks blocks.
constexpr int kPrefillRows = 128;
constexpr int kPrefillMaxBlocks = 4096;
// Shared-prefix decode cuts each group's prefix into at most kMaxPrefixSlices slices of at least
// kPrefixMinSplit tokens: enough workgroups to spread a short prefix over the GPU, and a bounded
// number of extra partial states for the merge to read.
constexpr int kMaxPrefixSlices = 4;
constexpr int kPrefixMinSplit = 128;
inline int prefix_split_tokens(int max_prefix_tokens) {
  int split = kPrefixMinSplit;
  while ((long long)split * kMaxPrefixSlices < max_prefix_tokens) split *= 2;
  return split;
}

struct PrefillParams {
  _Float16* out;
  const _Float16* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [S + 1] first query row of each sequence, then the total
  int32_t num_tokens;          // rows of q and out
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t max_query_len;
  int32_t max_context_len;
  int32_t group;
  int32_t q_tiles;             // ceil(max_query_len * group / kPrefillRows)
  float scale_log2;
  // Prefix pass of shared-prefix decode: the "sequences" are groups, query_start is the group
  // ranges over decode sequences, group_prefix_blocks[g] the shared leading blocks (read from
  // the first member's table row), and the unnormalised partial of each (member, query head)
  // goes to slot 0 of the decode workspace instead of a normalised output.
  const int32_t* group_prefix_blocks;
  float* ws_ml;
  float* ws_acc;
  int32_t part_slots;
  int32_t max_prefix_blocks;
  int32_t prefix_split;
  int32_t prefix_slices;  // grid slices per group: ceil(max_prefix_blocks * BS / prefix_split)
};

// Launchers: return hipSuccess or the launch error. Arguments are already validated.
hipError_t launch_decode(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                         int head_tile, bool kv_fp8, hipStream_t stream);
hipError_t launch_decode_append(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                                int head_tile, bool kv_fp8, hipStream_t stream);
hipError_t launch_decode_mfma_append(const DecodeParams& p, int num_seqs, int head_dim,
                                     int block_size, int rows, bool kv_fp8, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                              int rows, bool kv_fp8, hipStream_t stream);
// Shared-prefix decode in one launch: n_prefix prefix-pass workgroups (f) and the vector-ALU
// decode grid (p, with deferred_merge = 2); launch_decode_merge must follow.
hipError_t launch_shared_prefix_decode(const DecodeParams& p, const PrefillParams& f,
                                       int n_prefix, int num_seqs, int head_dim, int block_size,
                                       int head_tile, bool kv_fp8, bool append,
                                       hipStream_t stream);
// Merge of the partition partials of every sequence that spans more than one partition (after a
// decode launch with deferred_merge = 1, on the same stream), and with deferred_merge = 2 also
// of every sequence that has prefix partials.
hipError_t launch_decode_merge(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                               hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int num_seqs, int head_dim, int block_size,
                          bool kv_fp8, hipStream_t stream);
hipError_t launch_prefix_pass(const PrefillParams& p, int num_groups, int head_dim, int block_size,
                              bool kv_fp8, hipStream_t stream);
hipError_t launch_kv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, hipStream_t stream);
hipError_t launch_kv_write_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                               float* k_scale, float* v_scale, const int64_t* slot_mapping,
                               int num_tokens, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_mapping, int num_pairs, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, int elem_bytes,
                              hipStream_t stream);
hipError_t launch_swap_blocks(const void* src_k, const void* src_v, const float* src_ks,
                              const float* src_vs, void* dst_k, void* dst_v, float* dst_ks,
                              float* dst_vs, const int32_t* block_mapping, int num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int src_blocks,
                              int dst_blocks, int elem_bytes, hipStream_t stream);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace pa

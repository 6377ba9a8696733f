// C-ABI entry points: host-side validation, grid sizing and launch on the caller's stream.
// Nothing here allocates, frees or synchronises; all buffers belong to the caller.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.hpp"

// Decode workspace of pa_decode_append_noalloc: each GPU the library runs on holds its own copy
// for the life of the process (16 MiB, PA_NOALLOC_SCRATCH_BYTES in pa.h).
constexpr size_t kScratchBytes = size_t(16) << 20;
static_assert(kScratchBytes % pa::kWsGranule == 0, "whole workspace granules");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }
bool supported_block_size(int bs) { return bs == 8 || bs == 16 || bs == 32 || bs == 64; }
bool known_dtype(int t) { return t == PA_KV_F16 || t == PA_KV_FP8_E4M3; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_last_hip_error = static_cast<int>(e);
  return PA_ERR_HIP;
}

// Resolves the partition size (0 = automatic) and the grid's partition count; false if invalid.
// `prefix`: shared-prefix decode, whose kernel choice (and so automatic size) can differ.
bool resolve_partition(int num_seqs, int num_q_heads, int num_kv_heads, int block_size,
                       bool kv8, bool prefix, long long max_ctx, int partition_tokens,
                       int* part_tokens, int* max_parts) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_ctx > (1LL << 30)) return false;
  const int group = num_q_heads / num_kv_heads;
  const int units_per_seq = num_kv_heads * (group / pa::decode_rows(group, kv8, prefix));
  const int ctx = (int)(max_ctx > 0 ? max_ctx : 1);
  int pt = partition_tokens;
  if (pt == 0)
    pt = pa::auto_part_tokens(num_seqs, units_per_seq, ctx, block_size,
                              pa::decode_target_units(group, prefix),
                              pa::decode_single_units(group, prefix));
  if (!pa::valid_part_tokens(pt, block_size)) return false;
  const long long parts = pa::ceil_div(ctx, pt);
  if (parts > 65535) return false;
  *part_tokens = pt;
  *max_parts = (int)parts;
  return true;
}

// ---- library-owned decode workspace for callers that cannot allocate ---------------------
// `scratch` (file scope, above) serves as the decode workspace of pa_decode_append_noalloc.
// In host code its name is only a stand-in: the device address, different on every GPU, comes
// from hipGetSymbolAddress with that GPU current, once per device, and only that address is used.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch; on the first call on that GPU, also enqueues a
// clear of its counter zone on `stream` (before the caller's kernels, on the same stream).
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t es = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (es != hipSuccess) return hip_status(es);
    if (ptr == nullptr || !aligned(ptr, 256)) return PA_ERR_HIP;
    const int rc = hip_status(pa::launch_zero_fill(ptr, pa::ws_counter_zone(kScratchBytes), stream));
    if (rc != PA_OK) return rc;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim / block_size / dtype";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int pa_last_hip_error(void) { return g_last_hip_error; }

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                   int32_t kv_dtype, int32_t partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || !supported_head_dim(head_dim) ||
      !supported_block_size(block_size) || !known_dtype(kv_dtype) || max_context_len <= 0)
    return 0;
  int pt = 0, parts = 0;
  if (!resolve_partition(num_seqs, num_q_heads, num_kv_heads, block_size,
                         kv_dtype == PA_KV_FP8_E4M3, false, max_context_len,
                         partition_tokens, &pt, &parts))
    return 0;
  return pt;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t kv_dtype, int32_t partition_tokens) {
  const int pt = pa_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            block_size, max_context_len, kv_dtype,
                                            partition_tokens);
  if (pt == 0) return 0;
  const int group = num_q_heads / num_kv_heads;
  const int hg_total =
      num_kv_heads * (group / pa::decode_rows(group, kv_dtype == PA_KV_FP8_E4M3, false));
  return pa::workspace_layout(num_seqs, num_q_heads, hg_total, head_dim,
                              (int)pa::ceil_div(max_context_len, pt)).total;
}

}  // extern "C"

namespace {

// The new-token arguments of pa_decode_append (all null for the other decode entry points).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  float* k_scale_w;  // writable scales of an 8-bit cache
  float* v_scale_w;
};

// Shared body of pa_decode, pa_decode_shared_prefix (groups != nullptr) and pa_decode_append
// (app != nullptr).
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const float* k_scale, const float* v_scale, const int32_t* block_tables,
                const int32_t* context_lens, const int32_t* seq_order, const AppendArgs* app,
                const int32_t* group_start,
                const int32_t* group_prefix_blocks, int32_t num_groups, int32_t max_group_seqs,
                int32_t max_prefix_blocks, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                int32_t max_context_len, int32_t partition_tokens, float scale, int32_t kv_dtype,
                void* workspace, size_t workspace_bytes_given, void* stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (!known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  const bool fp8 = kv_dtype == PA_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(seq_order, 4) ||
      (fp8 && (!aligned(k_scale, 4) ||
      !aligned(v_scale, 4))))
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 65535) return PA_ERR_INVALID_ARG;
  if (app) {
    if (!app->k_new || !app->v_new || !app->slot_mapping || !aligned(app->k_new, 16) ||
        !aligned(app->v_new, 16) || !aligned(app->slot_mapping, 8))
      return PA_ERR_INVALID_ARG;
    if ((long long)num_blocks * block_size >= (1LL << 31)) return PA_ERR_INVALID_ARG;
    if ((long long)num_seqs * num_kv_heads * (head_dim * 2 / 16) >= (1LL << 31))
      return PA_ERR_INVALID_ARG;
  }
  const bool groups = group_start != nullptr;
  if (groups) {
    if (!group_prefix_blocks || !aligned(group_start, 4) || !aligned(group_prefix_blocks, 4) ||
        num_groups <= 0 || max_group_seqs <= 0 || max_group_seqs > num_seqs ||
        max_prefix_blocks <= 0)
      return PA_ERR_INVALID_ARG;
  }
  const long long max_ctx = max_context_len > 0 ? (long long)max_context_len
                                                : (long long)max_blocks_per_seq * block_size;
  if (max_ctx > (long long)max_blocks_per_seq * block_size || max_ctx > (1LL << 30))
    return PA_ERR_INVALID_ARG;
  int part_tokens = 0, max_parts = 0;
  if (!resolve_partition(num_seqs, num_q_heads, num_kv_heads, block_size, fp8, groups, max_ctx,
                         partition_tokens, &part_tokens, &max_parts))
    return partition_tokens != 0 ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG;
  const int group = num_q_heads / num_kv_heads;
  const int gt = pa::decode_rows(group, fp8, groups);
  const bool mfma = pa::decode_uses_mfma(group, groups);
  // prefix blocks beyond the clamp (table width, on-chip id list, host bound on contexts) are
  // simply decoded per sequence, so the clamp never changes the result
  int prefix_blocks = 0, prefix_split = 0, prefix_slices = 0;
  long long prefix_tiles = 0;
  if (groups) {
    prefix_blocks = (int)std::min<long long>(
        std::min<long long>(max_prefix_blocks, max_blocks_per_seq),
        std::min<long long>(pa::kPrefillMaxBlocks, max_ctx / block_size));
    prefix_split = pa::prefix_split_tokens(prefix_blocks * block_size);
    prefix_slices = (int)pa::ceil_div((long long)prefix_blocks * block_size, prefix_split);
    prefix_tiles = pa::ceil_div((long long)max_group_seqs * group, pa::kPrefillRows);
    if (prefix_tiles * num_kv_heads * num_groups * std::max(prefix_slices, 1) >= (1LL << 31))
      return PA_ERR_INVALID_ARG;
  }
  const int part_slots = max_parts + prefix_slices;
  const pa::WorkspaceLayout ws = pa::workspace_layout(num_seqs, num_q_heads,
                                                      num_kv_heads * (group / gt), head_dim,
                                                      part_slots);
  if (ws.total > 0 && (workspace == nullptr || !pa::workspace_fits(ws, workspace_bytes_given) ||
                       !aligned(workspace, 256)))
    return PA_ERR_WORKSPACE;

  pa::DecodeParams p{};
  p.out = static_cast<_Float16*>(out);
  p.q = static_cast<const _Float16*>(q);
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.seq_order = seq_order;
  char* wsb = static_cast<char*>(workspace);
  const size_t zone = pa::ws_counter_zone(workspace_bytes_given);
  p.counters = ws.total ? reinterpret_cast<int32_t*>(wsb) : nullptr;
  p.ws_ml = ws.total ? reinterpret_cast<float*>(wsb + zone + ws.ml_rel) : nullptr;
  p.ws_acc = ws.total ? reinterpret_cast<float*>(wsb + zone + ws.acc_rel) : nullptr;
  p.group_start = group_start;
  p.group_prefix_blocks = group_prefix_blocks;
  p.num_groups = groups ? num_groups : 0;
  p.max_prefix_blocks = prefix_blocks;
  p.prefix_split = prefix_split > 0 ? prefix_split : pa::kPrefixMinSplit;
  p.part_slots = part_slots;
  p.part_tokens = part_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.max_parts = max_parts;
  p.group = group;
  p.head_groups = group / gt;
  p.scale_log2 = scale * 1.4426950408889634f;
  // Split sequences of the vector-ALU kernel in batch order are merged by a kernel of its own
  // (block-size sweep at 128 x [32, 8192] tokens: 145 against 150 us with the last-arriving
  // workgroup merging). With a caller's dispatch order the last partitions go first and the
  // last-arriving workgroup merges in-kernel, inside the grid's tail (same lengths, longest
  // first: 136 against 139.5 us). The matrix-core kernel's workgroups always merge in-kernel
  // (MQA at 64 x 2,048 tokens: 20.5 against 22.2 us with the separate merge). Both merges take
  // the partials in the same order with the same arithmetic.
  p.deferred_merge = ws.total > 0 && max_parts > 1 && !mfma && seq_order == nullptr;
  // Matrix-core decode: cacheable K/V loads when the call reads at most 256 MiB of KV (the
  // Infinity Cache's size; bounded by num_seqs x max_context_len), non-temporal loads above.
  p.kv_cached = (long long)num_seqs * max_ctx * num_kv_heads * head_dim * (fp8 ? 1 : 2) * 2 <=
                (256LL << 20);
  // Shared prefixes with the vector-ALU decode: the prefix pass and the decode run in one launch
  // and every partial is merged by the merge kernel (shared-prefix step of 100 sequences: see
  // launch_shared_prefix_decode); with the matrix-core decode the prefix pass is a launch of its
  // own before it.
  const bool one_launch = groups && prefix_blocks > 0 && !mfma;
  if (one_launch) p.deferred_merge = 2;
  const hipStream_t st = static_cast<hipStream_t>(stream);

  pa::PrefillParams f{};
  if (groups && prefix_blocks > 0) {
    // prefix pass: every group's shared blocks once per KV head, for all member queries
    f.q = p.q;
    f.k_cache = p.k_cache;
    f.v_cache = p.v_cache;
    f.k_scale = k_scale;
    f.v_scale = v_scale;
    f.block_tables = block_tables;
    f.context_lens = context_lens;
    f.query_start = group_start;
    f.num_tokens = num_seqs;
    f.num_q_heads = num_q_heads;
    f.num_kv_heads = num_kv_heads;
    f.max_blocks_per_seq = max_blocks_per_seq;
    f.num_blocks = num_blocks;
    f.max_query_len = max_group_seqs;
    f.max_context_len = (int)(std::min<long long>(max_ctx / block_size, pa::kPrefillMaxBlocks) *
                              block_size);
    f.group = group;
    f.q_tiles = (int)prefix_tiles;
    f.scale_log2 = p.scale_log2;
    f.group_prefix_blocks = group_prefix_blocks;
    f.ws_ml = p.ws_ml;
    f.ws_acc = p.ws_acc;
    f.part_slots = part_slots;
    f.max_prefix_blocks = prefix_blocks;
    f.prefix_split = prefix_split;
    f.prefix_slices = prefix_slices;
    if (!one_launch) {
      const int rc = hip_status(pa::launch_prefix_pass(f, num_groups, head_dim, block_size, fp8, st));
      if (rc != PA_OK) return rc;
    }
  }
  if (one_launch) {
    const long long n_prefix = prefix_tiles * num_kv_heads * num_groups * prefix_slices;
    if (n_prefix + (long long)num_kv_heads * (group / gt) * num_seqs * max_parts >= (1LL << 31))
      return PA_ERR_INVALID_ARG;
    if (app && fp8) {
      // E4M3: the append kernel (with the block-scale policy) first
      const int rc = hip_status(pa::launch_kv_write_fp8(
          app->k_new, app->v_new, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
          app->k_scale_w, app->v_scale_w, app->slot_mapping, num_seqs, num_kv_heads, head_dim,
          block_size, num_blocks, st));
      if (rc != PA_OK) return rc;
    } else if (app) {
      p.k_new = static_cast<const uint8_t*>(app->k_new);
      p.v_new = static_cast<const uint8_t*>(app->v_new);
      p.slot_mapping = app->slot_mapping;
      p.k_cache_w = static_cast<uint8_t*>(const_cast<void*>(k_cache));
      p.v_cache_w = static_cast<uint8_t*>(const_cast<void*>(v_cache));
    }
    const hipError_t e = pa::launch_shared_prefix_decode(p, f, (int)n_prefix, num_seqs, head_dim,
                                                         block_size, gt, fp8, app && !fp8, st);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(pa::launch_decode_merge(p, num_seqs, head_dim, block_size, st));
  }
  if (app) {
    // One launch: the decode kernel stores and attends the new rows itself. For E4M3 caches it
    // also applies the block-scale policy when one head tile covers the KV head's query heads:
    // the last block of a (sequence, KV head) is then read by one workgroup only, the one that
    // re-encodes and stores it.
    if (!fp8 || group == gt) {
      p.k_new = static_cast<const uint8_t*>(app->k_new);
      p.v_new = static_cast<const uint8_t*>(app->v_new);
      p.slot_mapping = app->slot_mapping;
      p.k_cache_w = static_cast<uint8_t*>(const_cast<void*>(k_cache));
      p.v_cache_w = static_cast<uint8_t*>(const_cast<void*>(v_cache));
      p.k_scale_w = app->k_scale_w;
      p.v_scale_w = app->v_scale_w;
      const hipError_t e =
          mfma ? pa::launch_decode_mfma_append(p, num_seqs, head_dim, block_size, gt, fp8, st)
               : pa::launch_decode_append(p, num_seqs, head_dim, block_size, gt, fp8, st);
      if (e != hipSuccess || !p.deferred_merge) return hip_status(e);
      return hip_status(pa::launch_decode_merge(p, num_seqs, head_dim, block_size, st));
    }
    // the append kernel first (E4M3 caches: with the block-scale policy), then the decode
    const hipError_t e =
        fp8 ? pa::launch_kv_write_fp8(app->k_new, app->v_new, const_cast<void*>(k_cache),
                                      const_cast<void*>(v_cache), app->k_scale_w, app->v_scale_w,
                                      app->slot_mapping, num_seqs, num_kv_heads, head_dim,
                                      block_size, num_blocks, st)
            : pa::launch_kv_write(app->k_new, app->v_new, const_cast<void*>(k_cache),
                                  const_cast<void*>(v_cache), app->slot_mapping, num_seqs,
                                  num_kv_heads, head_dim, block_size, num_blocks, st);
    const int rc = hip_status(e);
    if (rc != PA_OK) return rc;
  }
  const hipError_t e = mfma
                           ? pa::launch_decode_mfma(p, num_seqs, head_dim, block_size, gt, fp8, st)
                           : pa::launch_decode(p, num_seqs, head_dim, block_size, gt, fp8, st);
  if (e != hipSuccess || !p.deferred_merge) return hip_status(e);
  return hip_status(pa::launch_decode_merge(p, num_seqs, head_dim, block_size, st));
}

}  // namespace

extern "C" {

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_tables,
              const int32_t* context_lens,
              const int32_t* seq_order, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
              int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_tokens,
              float scale, int32_t kv_dtype, void* workspace, size_t workspace_bytes_given,
              void* stream) {
  return decode_impl(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     seq_order, nullptr, nullptr, nullptr, 0, 0, 0, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                     partition_tokens, scale, kv_dtype, workspace, workspace_bytes_given, stream);
}

int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                     const int64_t* slot_mapping, const int32_t* block_tables,
                     const int32_t* context_lens,
              const int32_t* seq_order, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                     int32_t partition_tokens, float scale, int32_t kv_dtype, void* workspace,
                     size_t workspace_bytes_given, void* stream) {
  const AppendArgs app{k_new, v_new, slot_mapping, k_scale, v_scale};
  return decode_impl(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     seq_order, &app, nullptr, nullptr, 0, 0, 0, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                     partition_tokens, scale, kv_dtype, workspace, workspace_bytes_given, stream);
}

int pa_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             const int64_t* slot_mapping, const int32_t* block_tables,
                             const int32_t* context_lens,
              const int32_t* seq_order, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_context_len, int32_t partition_tokens, float scale,
                             int32_t kv_dtype, void* stream) {
  // the size check comes first, so an oversized call is rejected before anything touches the
  // device; pa_decode_workspace_bytes returns 0 for invalid arguments, which decode_impl then
  // reports itself
  const long long max_ctx = max_context_len > 0 ? (long long)max_context_len
                                                : (long long)max_blocks_per_seq * block_size;
  size_t need = 0;
  if (max_ctx > 0 && max_ctx <= (1LL << 30))
    need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     (int32_t)max_ctx, kv_dtype, partition_tokens);
  if (need > kScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (need > 0) {
    const int rc = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
    if (rc != PA_OK) return rc;
    ws_bytes = kScratchBytes;
  }
  const AppendArgs app{k_new, v_new, slot_mapping, k_scale, v_scale};
  return decode_impl(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     seq_order, &app, nullptr, nullptr, 0, 0, 0, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                     partition_tokens, scale, kv_dtype, ws, ws_bytes, stream);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t max_context_len,
                                               int32_t kv_dtype, int32_t partition_tokens) {
  // the shared-prefix call's own partition policy (its kernel choice can differ from pa_decode's)
  if (num_seqs <= 0 || num_q_heads <= 0 || !supported_head_dim(head_dim) ||
      !supported_block_size(block_size) || !known_dtype(kv_dtype) || max_context_len <= 0)
    return 0;
  const bool kv8 = kv_dtype == PA_KV_FP8_E4M3;
  int pt = 0, parts = 0;
  if (!resolve_partition(num_seqs, num_q_heads, num_kv_heads, block_size, kv8, true,
                         max_context_len, partition_tokens, &pt, &parts))
    return 0;
  const int group = num_q_heads / num_kv_heads;
  const int hg_total = num_kv_heads * (group / pa::decode_rows(group, kv8, true));
  return pa::workspace_layout(num_seqs, num_q_heads, hg_total, head_dim,
                              (int)pa::ceil_div(max_context_len, pt) + pa::kMaxPrefixSlices).total;
}

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
                            void* stream) {
  if (!group_start) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     seq_order, nullptr, group_start, group_prefix_blocks, num_groups, max_group_seqs,
                     max_prefix_blocks, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, partition_tokens, scale, kv_dtype,
                     workspace, workspace_bytes, stream);
}

int pa_decode_shared_prefix_append(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    float* k_scale, float* v_scale, const int64_t* slot_mapping, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* seq_order, const int32_t* group_start,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t max_group_seqs,
    int32_t max_prefix_blocks, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t partition_tokens, float scale, int32_t kv_dtype,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (!group_start) return PA_ERR_INVALID_ARG;
  const AppendArgs app{k_new, v_new, slot_mapping, k_scale, v_scale};
  return decode_impl(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     seq_order, &app, group_start, group_prefix_blocks, num_groups,
                     max_group_seqs, max_prefix_blocks, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                     partition_tokens, scale, kv_dtype, workspace, workspace_bytes, stream);
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const float* k_scale, const float* v_scale, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
               int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
               int32_t max_query_len, int32_t max_context_len, float scale, int32_t kv_dtype,
               void* stream) {
  if (num_seqs <= 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || max_query_len < 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (!known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  const bool fp8 = kv_dtype == PA_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return PA_ERR_INVALID_ARG;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size)
    return PA_ERR_INVALID_ARG;
  if ((long long)max_context_len > (long long)pa::kPrefillMaxBlocks * block_size)
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (max_query_len == 0) return PA_ERR_INVALID_ARG;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4) ||
      (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
    return PA_ERR_INVALID_ARG;
  const int group = num_q_heads / num_kv_heads;
  const long long q_tiles = pa::ceil_div((long long)max_query_len * group, pa::kPrefillRows);
  if (q_tiles * num_kv_heads * num_seqs >= (1LL << 31)) return PA_ERR_INVALID_ARG;

  pa::PrefillParams p{};
  p.out = static_cast<_Float16*>(out);
  p.q = static_cast<const _Float16*>(q);
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.num_tokens = num_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.max_query_len = max_query_len;
  p.max_context_len = max_context_len;
  p.group = group;
  p.q_tiles = (int)q_tiles;
  p.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(pa::launch_prefill(p, num_seqs, head_dim, block_size, fp8,
                                       static_cast<hipStream_t>(stream)));
}

int pa_kv_write(const void* k, const void* v, void* k_cache, void* v_cache, float* k_scale,
                float* v_scale, const int64_t* slot_mapping, int32_t num_tokens,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t kv_dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (!known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  const bool fp8 = kv_dtype == PA_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return PA_ERR_INVALID_ARG;
  if ((long long)num_blocks * block_size >= (1LL << 31)) return PA_ERR_INVALID_ARG;
  if ((long long)num_tokens * num_kv_heads * (head_dim * 2 / 16) >= (1LL << 31))
    return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8) || (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
    return PA_ERR_INVALID_ARG;
  if (fp8)
    return hip_status(pa::launch_kv_write_fp8(k, v, k_cache, v_cache, k_scale, v_scale,
                                              slot_mapping, num_tokens, num_kv_heads, head_dim,
                                              block_size, num_blocks,
                                              static_cast<hipStream_t>(stream)));
  return hip_status(pa::launch_kv_write(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                        num_kv_heads, head_dim, block_size, num_blocks,
                                        static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int32_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                   void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (!known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if ((long long)num_blocks * block_size >= (1LL << 31)) return PA_ERR_INVALID_ARG;
  if (num_kv_heads > 65535) return PA_ERR_INVALID_ARG;
  const bool fp8 = kv_dtype == PA_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_mapping, 4))
    return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, k_scale, v_scale, block_mapping,
                                           num_pairs, num_kv_heads, head_dim, block_size,
                                           num_blocks, fp8 ? 1 : 2,
                                           static_cast<hipStream_t>(stream)));
}

int pa_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scale,
                   const float* src_v_scale, void* dst_k, void* dst_v, float* dst_k_scale,
                   float* dst_v_scale, const int32_t* block_mapping, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t src_num_blocks, int32_t dst_num_blocks, int32_t kv_dtype,
                   void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (!known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > pa::kThreads) return PA_ERR_UNSUPPORTED;
  const bool fp8 = kv_dtype == PA_KV_FP8_E4M3;
  const bool scales[4] = {src_k_scale != nullptr, src_v_scale != nullptr, dst_k_scale != nullptr,
                          dst_v_scale != nullptr};
  for (bool s : scales)
    if (s != fp8) return PA_ERR_INVALID_ARG;
  const long long block_bytes = (long long)num_kv_heads * block_size * head_dim * (fp8 ? 1 : 2);
  if ((long long)src_num_blocks * block_bytes / 16 >= (1LL << 40) || block_bytes / 16 >= (1LL << 31))
    return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) ||
      !aligned(block_mapping, 4))
    return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_swap_blocks(src_k, src_v, src_k_scale, src_v_scale, dst_k, dst_v,
                                           dst_k_scale, dst_v_scale, block_mapping, num_pairs,
                                           num_kv_heads, head_dim, block_size, src_num_blocks,
                                           dst_num_blocks, fp8 ? 1 : 2,
                                           static_cast<hipStream_t>(stream)));
}

int pa_decode_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  const size_t zone = pa::ws_counter_zone(workspace_bytes);
  if (zone == 0) return PA_OK;  // too small to hold counters: nothing to clear
  if (!workspace || !aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_zero_fill(workspace, zone, static_cast<hipStream_t>(stream)));
}

int pa_stream_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || !aligned(buf, 16) || !aligned(sink, 4)) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_stream_read(buf, bytes, static_cast<uint32_t*>(sink),
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

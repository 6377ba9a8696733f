// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// ---- decode geometry -------------------------------------------------------------------
// A workgroup of kWaves wavefronts owns one (sequence, KV-head group, context partition) and
// processes kPartTokens consecutive logical tokens; each wave owns kWaveTokens of them and walks
// them in tiles of kTileTokens (four 16-lane rows x four steps of one token per row).
constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kRows = 4;
constexpr int kSteps = 4;
constexpr int kTileTokens = kRows * kSteps;
constexpr int kPartTokens = 512;
constexpr int kWaveTokens = kPartTokens / kWaves;
constexpr int kTilesPerWave = kWaveTokens / kTileTokens;

struct DecodeParams {
  _Float16* out;
  const _Float16* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_ml;   // [S, Hq, max_parts, 2] (running max in log2 units, running sum)
  float* ws_acc;  // [S, Hq, max_parts, D] unnormalised weighted value sums
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t max_parts;
  int32_t group;        // G = Hq / Hkv
  int32_t head_groups;  // G / GT workgroups per KV head
  float scale_log2;     // softmax scale * log2(e)
};

// Largest compiled query-head tile (GT) dividing the group size G.
inline int pick_head_tile(int group) {
  for (int gt : {8, 4, 2, 1})
    if (group % gt == 0) return gt;
  return 1;
}

inline int decode_num_parts(int max_context_len) {
  return max_context_len <= 0 ? 1 : (max_context_len + kPartTokens - 1) / kPartTokens;
}

// Launchers: return hipSuccess or the launch error. Arguments are already validated.
hipError_t launch_decode(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                         int head_tile, bool kv_fp8, hipStream_t stream);
hipError_t launch_kv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_mapping, int num_pairs, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, int elem_bytes,
                              hipStream_t stream);

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace pa

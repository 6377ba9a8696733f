// Cache updates of a decode step for gfx950: slot-mapped append and copy-on-write block copy.
//
// * kv_write: a new token's key and value go to the slot the host chose for it, slot =
//   block * BS + offset ("vLLM의 핵심 이해: PagedAttention", section 6: each token maps to a
//   page and a position inside it). One thread moves one 16-byte chunk of one (token, head)
//   row, so a wave writes 4 rows of 256 B (D = 128) with fully coalesced stores.
// * copy_blocks: before a sequence writes into a shared block that is still filling, that
//   block is copied into a private block ("serving-paged-attention", section "공유는 표를
//   베끼는 일이 된다"). In the [NB, Hkv, BS, D] layout every (block, head) tile is one
//   contiguous run of BS * D elements, so a workgroup per (pair, head) streams it with 16-byte
//   loads and stores; per-(block, head) scales of an 8-bit cache travel with it.
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(256) void kv_write_kernel(const uint4* __restrict__ k,
                                                       const uint4* __restrict__ v,
                                                       uint4* __restrict__ k_cache,
                                                       uint4* __restrict__ v_cache,
                                                       const int64_t* __restrict__ slot_mapping,
                                                       int num_rows, int num_kv_heads,
                                                       int chunks_per_row, int block_size,
                                                       int64_t num_slots) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = gid / chunks_per_row;  // (token, head) row
  if (row >= num_rows) return;
  const int c = gid - row * chunks_per_row;
  const int t = row / num_kv_heads;
  const int h = row - t * num_kv_heads;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped token, or out of range: no write
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + off) * chunks_per_row + c;
  const size_t src = (size_t)row * chunks_per_row + c;
  k_cache[dst] = k[src];
  v_cache[dst] = v[src];
}

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, float* __restrict__ k_scale,
    float* __restrict__ v_scale, const int32_t* __restrict__ block_mapping, int num_kv_heads,
    int chunks_per_tile, int num_blocks) {
  const int pair = blockIdx.x;
  const int h = blockIdx.y;
  const int src = block_mapping[2 * pair];
  const int dst = block_mapping[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;  // out of range: skipped
  const size_t s0 = ((size_t)src * num_kv_heads + h) * chunks_per_tile;
  const size_t d0 = ((size_t)dst * num_kv_heads + h) * chunks_per_tile;
  for (int c = threadIdx.x; c < chunks_per_tile; c += kCopyThreads) {
    const uint4 kv = k_cache[s0 + c];
    const uint4 vv = v_cache[s0 + c];
    k_cache[d0 + c] = kv;
    v_cache[d0 + c] = vv;
  }
  if (threadIdx.x == 0 && k_scale != nullptr) {
    k_scale[(size_t)dst * num_kv_heads + h] = k_scale[(size_t)src * num_kv_heads + h];
    v_scale[(size_t)dst * num_kv_heads + h] = v_scale[(size_t)src * num_kv_heads + h];
  }
}

}  // namespace

hipError_t launch_kv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, hipStream_t stream) {
  const int chunks_per_row = head_dim * 2 / 16;
  const int num_rows = num_tokens * num_kv_heads;
  const long long threads = (long long)num_rows * chunks_per_row;
  const int blocks = (int)((threads + 255) / 256);
  kv_write_kernel<<<blocks, 256, 0, stream>>>(
      static_cast<const uint4*>(k), static_cast<const uint4*>(v), static_cast<uint4*>(k_cache),
      static_cast<uint4*>(v_cache), slot_mapping, num_rows, num_kv_heads, chunks_per_row,
      block_size, (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_mapping, int num_pairs, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, int elem_bytes,
                              hipStream_t stream) {
  const int chunks_per_tile = block_size * head_dim * elem_bytes / 16;
  copy_blocks_kernel<<<dim3(num_pairs, num_kv_heads), kCopyThreads, 0, stream>>>(
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), k_scale, v_scale,
      block_mapping, num_kv_heads, chunks_per_tile, num_blocks);
  return hipGetLastError();
}

}  // namespace pa

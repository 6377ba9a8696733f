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
#include "fp8_append.hpp"
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
  // the row's data and its slot are loaded together (one memory round trip, not two)
  const size_t src = (size_t)row * chunks_per_row + c;
  const uint4 kx = k[src];
  const uint4 vx = v[src];
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped token, or out of range: no write
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + off) * chunks_per_row + c;
  k_cache[dst] = kx;
  v_cache[dst] = vx;
}

// ---- append into an 8-bit (OCP E4M3) cache --------------------------------------------------
// The block-scale policy and the encoding are in fp8_append.hpp. Tokens of one call that land
// in the same block are applied in call order (they must be consecutive in the call: a decode
// step's single token, or a prefill chunk's tokens in order); sequences never write into a
// shared block.
// Launched with two waves per (token, KV head): wave 0 appends K, wave 1 appends V (each cache
// has its own scales, so the two are independent and run side by side).
template <int D>
__global__ __launch_bounds__(128) void kv_write_fp8_kernel(
    const _Float16* __restrict__ k, const _Float16* __restrict__ v, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int block_size,
    int64_t num_slots) {
  constexpr int PER = D / 64;  // bytes (elements) a lane owns in every row: 2 (D 128) or 1 (D 64)
  const int t0 = blockIdx.x / num_kv_heads;
  const int h = blockIdx.x - t0 * num_kv_heads;
  const int64_t slot0 = slot_mapping[t0];
  if (slot0 < 0 || slot0 >= num_slots) return;
  const int64_t blk = slot0 / block_size;
  // Consecutive tokens of the call that land in one block form a run; the workgroup of the
  // run's first token applies them in order, K in one wave and V in the other (the scale policy
  // is sequential within a block).
  if (t0 > 0) {
    const int64_t sp = slot_mapping[t0 - 1];
    if (sp >= 0 && sp < num_slots && sp / block_size == blk) return;
  }
  const int lane = threadIdx.x & 63;
  const int which = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    uint8_t* tile = (which == 0 ? k_cache : v_cache) + ((size_t)blk * num_kv_heads + h) * block_size * D;
    float* sc = (which == 0 ? k_scale : v_scale) + (size_t)blk * num_kv_heads + h;
    const _Float16* src = which == 0 ? k : v;
    // The block's scale is carried through the run in a (wave-uniform) register, and every lane
    // only ever touches its own PER bytes of each row, so no lane reads what another wrote.
    // The block's stored scale and the next token's slot are loaded before they are needed, so
    // each token costs one memory round trip.
    const float s_stored = *sc;
    float s_cur = 0.f;
    int64_t slot = slot0;
    for (int t = t0; t < num_tokens; ++t) {
      if (t > t0 && (slot < 0 || slot >= num_slots || slot / block_size != blk)) break;
      const int64_t next = t + 1 < num_tokens ? slot_mapping[t + 1] : -1;
      const int off = (int)(slot - blk * block_size);
      const _Float16* row = src + ((size_t)t * num_kv_heads + h) * D;
      float x[PER];
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        x[e] = (float)row[lane * PER + e];
        amax = fmaxf(amax, fabsf(x[e]));
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      const float s_prev = off == 0 ? 0.f : (t == t0 ? s_stored : s_cur);
      const float s = fp8_append_scale(amax, s_prev);
      if (s != s_prev && off > 0) {
        // re-encode the codes already in the block (this lane's bytes of rows 0 .. off-1)
        for (int r = 0; r < off; ++r) {
          uint8_t* p = tile + (size_t)r * D + lane * PER;
          if constexpr (PER == 2) {
            const uint32_t w = *reinterpret_cast<const uint16_t*>(p);
            const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
            *reinterpret_cast<uint16_t*>(p) = (uint16_t)(enc_pair<false>(
                fp8_rescaled(c.x, s_prev, s), fp8_rescaled(c.y, s_prev, s), 0u) & 0xFFFFu);
          } else {
            const uint32_t w = *p;
            const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
            *p = (uint8_t)(enc_pair<false>(fp8_rescaled(c.x, s_prev, s), 0.f, 0u) & 0xFFu);
          }
        }
      }
      uint8_t* dst = tile + (size_t)off * D + lane * PER;
      if constexpr (PER == 2) {
        const uint32_t o = enc_pair<false>(x[0] / s, x[1] / s, 0u);
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(o & 0xFFFFu);
      } else {
        const uint32_t o = enc_pair<false>(x[0] / s, 0.f, 0u);
        *dst = (uint8_t)(o & 0xFFu);
      }
      s_cur = s;
      slot = next;
    }
    if (lane == 0) *sc = s_cur;
  }
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

// Swap of whole blocks between two pools (device memory, or pinned host memory mapped into the
// device's address space): preemption by swap moves a request's blocks to host memory and later
// back ("serving-paged-attention", section "그래도 넘칠 때 — 선점"). In the [NB, Hkv, BS, D]
// layout a block of all KV heads is one contiguous run, so a workgroup per pair streams it
// with 16-byte loads and stores; the per-(block, head) scales of an 8-bit cache move with it.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
    const float* __restrict__ src_ks, const float* __restrict__ src_vs, uint4* __restrict__ dst_k,
    uint4* __restrict__ dst_v, float* __restrict__ dst_ks, float* __restrict__ dst_vs,
    const int32_t* __restrict__ block_mapping, int num_kv_heads, int chunks_per_block,
    int src_blocks, int dst_blocks) {
  const int pair = blockIdx.x;
  const int src = block_mapping[2 * pair];
  const int dst = block_mapping[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;  // out of range: skipped
  const size_t s0 = (size_t)src * chunks_per_block;
  const size_t d0 = (size_t)dst * chunks_per_block;
  for (int c = threadIdx.x; c < chunks_per_block; c += kCopyThreads) {
    const uint4 kv = src_k[s0 + c];
    const uint4 vv = src_v[s0 + c];
    dst_k[d0 + c] = kv;
    dst_v[d0 + c] = vv;
  }
  if (src_ks != nullptr && (int)threadIdx.x < num_kv_heads) {
    dst_ks[(size_t)dst * num_kv_heads + threadIdx.x] = src_ks[(size_t)src * num_kv_heads + threadIdx.x];
    dst_vs[(size_t)dst * num_kv_heads + threadIdx.x] = src_vs[(size_t)src * num_kv_heads + threadIdx.x];
  }
}

// Zero fill of a 16-byte aligned range with vector stores (a kernel rather than a memset
// node, so that a caller may capture it in a graph): clears the arrival counters of a decode
// workspace.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, const float* src_ks,
                              const float* src_vs, void* dst_k, void* dst_v, float* dst_ks,
                              float* dst_vs, const int32_t* block_mapping, int num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int src_blocks,
                              int dst_blocks, int elem_bytes, hipStream_t stream) {
  const int chunks = num_kv_heads * block_size * head_dim * elem_bytes / 16;
  swap_blocks_kernel<<<num_pairs, kCopyThreads, 0, stream>>>(
      static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v), src_ks, src_vs,
      static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), dst_ks, dst_vs, block_mapping,
      num_kv_heads, chunks, src_blocks, dst_blocks);
  return hipGetLastError();
}

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

hipError_t launch_kv_write_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                               float* k_scale, float* v_scale, const int64_t* slot_mapping,
                               int num_tokens, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, hipStream_t stream) {
  const int grid = num_tokens * num_kv_heads;
  const int64_t slots = (int64_t)num_blocks * block_size;
  auto kk = static_cast<const _Float16*>(k);
  auto vv = static_cast<const _Float16*>(v);
  auto kc = static_cast<uint8_t*>(k_cache);
  auto vc = static_cast<uint8_t*>(v_cache);
  if (head_dim == 128)
    kv_write_fp8_kernel<128><<<grid, 128, 0, stream>>>(kk, vv, kc, vc, k_scale, v_scale,
                                                      slot_mapping, num_tokens, num_kv_heads,
                                                      block_size, slots);
  else
    kv_write_fp8_kernel<64><<<grid, 128, 0, stream>>>(kk, vv, kc, vc, k_scale, v_scale,
                                                     slot_mapping, num_tokens, num_kv_heads,
                                                     block_size, slots);
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

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int blocks = (int)(want < 1024 ? want : 1024);
  zero_fill_kernel<<<blocks, 256, 0, stream>>>(static_cast<uint4*>(p), n);
  return hipGetLastError();
}

}  // namespace pa

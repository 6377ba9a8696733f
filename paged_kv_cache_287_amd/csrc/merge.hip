// Merge of split-context partials by a kernel of its own (decode launched with
// deferred_merge = 1).
//
// A sequence whose context spans several partitions leaves one unnormalised partial per
// partition (running max m_p in log2 units, running sum l_p, weighted value sum a_p), plus the
// prefix slices a shared-prefix pass stored before them. Partial softmax states combine without
// approximation (talk summary, FlashAttention paragraph):
//     out = sum_p 2^(m_p - M) a_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p.
// One thread merges 8 consecutive dims of one (sequence, query head) row, so its output is one
// 16-byte store and its value loads are two 16-byte loads per slot; the slots are taken 8 at a
// time with all their loads in flight, merged into a running (max, sum, value) in slot order,
// the same arithmetic as the in-kernel merge of the last-arriving workgroup. Sequences that fit
// one partition were written by the decode kernel itself and are skipped (their first-chunk
// loads, issued before the slot count is known, read stale slots and are discarded).
#include "decode_common.hpp"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int block_size) {
  constexpr int TPR = D / 8;  // threads per row
  const int b = blockIdx.y;
  const int row = (int)((blockIdx.x * 256u + threadIdx.x) / TPR);  // query head
  if (row >= p.num_q_heads) return;
  const int d0 = (int)(threadIdx.x % TPR) * 8;
  constexpr int kChunk = 8;
  typedef f32x4 f32x4x2[2];

  // The first chunk of slots is loaded before the slot count is known (in bounds: slot indices
  // are clamped to the row's part_slots), so those loads and the context length travel together.
  const size_t row0 = ((size_t)b * p.num_q_heads + row) * p.part_slots;
  const float* ml = p.ws_ml + row0 * 2;
  const float* ac = p.ws_acc + row0 * D + d0;
  float mv0[kChunk], lv0[kChunk];
  f32x4x2 av0[kChunk];
#pragma unroll
  for (int j = 0; j < kChunk; ++j) {
    const int i = min(j, p.part_slots - 1);
    mv0[j] = ml[2 * i];
    lv0[j] = ml[2 * i + 1];
    av0[j][0] = *reinterpret_cast<const f32x4*>(ac + (size_t)i * D);
    av0[j][1] = *reinterpret_cast<const f32x4*>(ac + (size_t)i * D + 4);
  }

  // the decode kernel's partition count for this sequence (see seq_range)
  const int L = p.context_lens[b];
  int start = 0, extra = 0;
  if (p.group_start != nullptr) {
    int lo = 0, hi = p.num_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.group_start[mid] <= b) lo = mid;
      else hi = mid - 1;
    }
    const bool member = p.group_start[lo] <= b && b < p.group_start[lo + 1];
    const int pb = member ? min(p.group_prefix_blocks[lo], p.max_prefix_blocks) : 0;
    if (pb > 0) {
      start = min(pb * block_size, max(L, 0));
      extra = (pb * block_size + p.prefix_split - 1) / p.prefix_split;
    }
  }
  const int span = L - start;
  const int nparts =
      min(span > 0 ? (span + p.part_tokens - 1) / p.part_tokens : 1, p.max_parts);
  // sequences the decode kernel finished itself: one partition and no prefix partial, or (prefix
  // pass in an earlier launch) one partition merged there with the prefix partials
  if (nparts == 1 && (extra == 0 || p.deferred_merge != 2)) return;
  const int nslots = nparts + extra;

  float mx = kNegInf, ls = 0.f, a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = 0.f;
  for (int i0 = 0; i0 < nslots; i0 += kChunk) {
    float mv[kChunk], lv[kChunk];
    f32x4 av[kChunk][2];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const bool in = i0 + j < nslots;
      if (i0 == 0) {
        // slots past nslots may hold anything (even non-finite values): zero weight and zeros
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        mv[j] = in ? mv0[j] : kNegInf;
        lv[j] = in ? lv0[j] : 0.f;
        av[j][0] = in ? av0[j][0] : z;
        av[j][1] = in ? av0[j][1] : z;
      } else {
        const int i = in ? i0 + j : i0;
        mv[j] = in ? ml[2 * i] : kNegInf;
        lv[j] = ml[2 * i + 1];
        av[j][0] = *reinterpret_cast<const f32x4*>(ac + (size_t)i * D);
        av[j][1] = *reinterpret_cast<const f32x4*>(ac + (size_t)i * D + 4);
      }
    }
    float mc = mx;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) mc = fmaxf(mc, mv[j]);
    const float r = fexp2(mx - mc);  // mx = -inf only before the first chunk: r = 0
    ls *= r;
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] *= r;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const float w = fexp2(mv[j] - mc);
      ls = fmaf(w, lv[j], ls);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = fmaf(w, av[j][0][u], a[u]);
        a[4 + u] = fmaf(w, av[j][1][u], a[4 + u]);
      }
    }
    mx = mc;
  }
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  h8 o;
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = (_Float16)(a[u] / ls);
  *reinterpret_cast<h8*>(p.out + ((size_t)b * p.num_q_heads + row) * D + d0) = o;
}

}  // namespace

hipError_t launch_decode_merge(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                               hipStream_t stream) {
  const int tpr = head_dim / 8;
  const dim3 grid((unsigned)((p.num_q_heads * tpr + 255) / 256), (unsigned)num_seqs);
  if (head_dim == 128) decode_merge_kernel<128><<<grid, 256, 0, stream>>>(p, block_size);
  else if (head_dim == 64) decode_merge_kernel<64><<<grid, 256, 0, stream>>>(p, block_size);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa

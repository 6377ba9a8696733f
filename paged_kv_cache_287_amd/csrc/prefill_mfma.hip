// Paged prefill for gfx950: causal attention of a chunk of new tokens over each sequence's paged
// KV cache, on matrix cores.
//
// Prefill is the compute-bound phase: the prompt is processed with large matrix products, while
// decode is bound by reading the cache ("LLM 추론 확장, 품질·비용 절충 필수", prefill and decode
// paragraphs). A chunk's keys and values are appended to the cache first (pa_kv_write); query j
// of a chunk of n then sits at position L - n + j and attends to positions 0 .. L - n + j, read
// through the block table ("serving-paged-attention", section "블록으로 쪼개고 표로 잇는다").
//
// Work decomposition. The query rows of one (sequence, KV head) are the chunk's tokens times the
// G query heads of that KV head, flattened as row = j * G + (h mod G). A workgroup of four waves
// owns 128 consecutive rows; each wave owns 32 of them (two 16-row MFMA tiles) for the whole
// attended range, so no cross-wave merge is needed. The workgroup walks the attended tokens in
// 64-token tiles; every tile of K and V is read from the cache once per workgroup, converted to
// fp16 if the cache is 8-bit, and staged in LDS for all four waves:
//   * K as [token][d] rows: a wave reads its MFMA A operand (16 tokens x 32 dims) straight out;
//   * V as [token][d] rows as well; the MFMA A operand V^T (a lane's eight contraction slots of
//     one dim) comes out of the transposed LDS read of gfx950 (ds_read_b64_tr_b16), two per
//     operand.
// Per tile and 16-row tile a wave forms S^T = K Q^T with v_mfma_f32_16x16x32_f16 (a lane ends up
// with four consecutive tokens of one row), updates that row's online softmax in log2 units, and
// accumulates O^T += V^T P^T, again with 16x16x32, where P^T is taken as-is from the lanes that
// computed it. Loads of the next tile are in flight while the current one is computed: for an
// fp16 cache they are gfx950's direct global -> LDS loads into the second of two tile buffers
// (one barrier per tile, no staging registers), for an 8-bit cache register loads that are
// converted and written to the one padded buffer between two barriers.
#include "prefill_body.hpp"

namespace pa {
namespace {

using pf::kTileTok;
using pf::prefill_body;
using pf::prefill_lds_bytes;

template <int D, int BS, bool KV8, bool PREFIX>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) {
  __shared__ __align__(16) uint8_t lds[prefill_lds_bytes<D, KV8, PREFIX>()];
  prefill_body<D, BS, KV8, PREFIX>(p, blockIdx.x, gridDim.x, lds);
}

template <int D, int BS, bool KV8, bool PREFIX>
hipError_t launch_one(const PrefillParams& p, long long workgroups, hipStream_t stream) {
  prefill_kernel<D, BS, KV8, PREFIX><<<dim3((unsigned)workgroups), kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, bool KV8, bool PREFIX>
hipError_t dispatch_bs(const PrefillParams& p, long long wgs, int bs, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_one<D, 8, KV8, PREFIX>(p, wgs, stream);
    case 16: return launch_one<D, 16, KV8, PREFIX>(p, wgs, stream);
    case 32: return launch_one<D, 32, KV8, PREFIX>(p, wgs, stream);
    case 64: return launch_one<D, 64, KV8, PREFIX>(p, wgs, stream);
  }
  return hipErrorInvalidValue;
}

template <bool PREFIX>
hipError_t dispatch(const PrefillParams& p, int num_units, int head_dim, int block_size,
                    bool kv_fp8, hipStream_t stream) {
  const long long wgs = (long long)p.q_tiles * p.num_kv_heads * num_units;
  if (head_dim == 128)
    return kv_fp8 ? dispatch_bs<128, true, PREFIX>(p, wgs, block_size, stream)
                  : dispatch_bs<128, false, PREFIX>(p, wgs, block_size, stream);
  if (head_dim == 64)
    return kv_fp8 ? dispatch_bs<64, true, PREFIX>(p, wgs, block_size, stream)
                  : dispatch_bs<64, false, PREFIX>(p, wgs, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int num_seqs, int head_dim, int block_size,
                          bool kv_fp8, hipStream_t stream) {
  return dispatch<false>(p, num_seqs, head_dim, block_size, kv_fp8, stream);
}

hipError_t launch_prefix_pass(const PrefillParams& p, int num_groups, int head_dim, int block_size,
                              bool kv_fp8, hipStream_t stream) {
  return dispatch<true>(p, num_groups * p.prefix_slices, head_dim, block_size, kv_fp8, stream);
}

}  // namespace pa

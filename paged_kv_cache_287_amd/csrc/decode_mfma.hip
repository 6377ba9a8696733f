// Paged decode attention for query groups of G >= 4 query heads per KV head (GQA-4 and wider,
// MQA; G >= 5 in shared-prefix decode) on gfx950 matrix cores.
//
// With G query heads sharing one KV head ("LLM 추론 확장, 품질·비용 절충 필수", attention-heads
// paragraph: MQA lets every query head share a single KV head) the per-token work is G dot
// products against each K row and G weighted sums of each V row: 32 flop per KV byte at G = 32,
// above what the VALU can sustain at HBM speed. Stacking the G query rows makes QK^T and PV
// dense 16-row tiles, so they run on MFMA:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_f16: A = a 16-token K tile in the operand layout
//     (lane l: token l%16, 8 consecutive dims of a 32-dim step). An fp16 tile is loaded in
//     whole rows and passes through a per-wave LDS tile into that layout; an 8-bit tile is
//     loaded straight in it (16 bytes per lane, two steps). B = the query rows, in registers. Lane l then owns query row l%16 and the scores of
//     tokens 4(l/16)..4(l/16)+3, so the online softmax (running max / sum per row, as in the
//     FlashAttention paragraph of the same talk summary) needs only two cross-row exchanges.
//   * O^T += V^T P^T with v_mfma_f32_16x16x16_f16: B = P^T is exactly the probabilities each
//     lane just computed (converted to fp16); A = V^T comes from a per-wave LDS tile. fp16: the
//     tile is stored transposed ([dim][token]): each lane loads 4 (or 2) consecutive tokens of
//     one 8-dim chunk of V and stores them as one 8-byte write per dim, and the operand (4
//     tokens of one dim) is one 8-byte read. E4M3: each lane loads 16 codes of one row (whole
//     rows per load instruction), stores them converted as fp16 rows, and the operand comes
//     out of gfx950's transposed LDS read (ds_read_b64_tr_b16). The accumulator lane l holds
//     row l%16, so rescaling by the running max is lane-local.
// Groups that are not a multiple of 16 fill 16- or 32-row tiles with padding rows of zero
// queries: the matrix cores still do the dot products for less VALU time than the VALU kernel's
// dot2 chains (GQA-8 at 64 x 2,048 tokens: 51 us against 76 us for fp16 KV, 45 against 64 for
// E4M3; GQA-4 in one 16-row tile, 4 rows real: the 8B shape 161.5 against 165.5-168 us, and
// 64 x 2,048 tokens with E4M3 47.5 against 57-63 us).
// Everything else (partitioning, block-id walk, double-buffered loads, fp8 scales,
// merge through LDS, partial publish / last-arrival merge, the fused append) follows the VALU
// kernel. For the fused append the new K/V rows of the workgroup's (sequence, KV head) are
// staged once in LDS (512 bytes at D 128), where the lanes of position L - 1 read them in the
// last tile: holding them in registers would cost the 16-row tile a wave per SIMD. With an 8-bit
// cache (one workgroup per KV head) wave 0 first applies the block-scale policy to them and
// stages codes; the tiles of the last block take the masked path, where a grown scale
// re-encodes the earlier codes as they are read and the appending workgroup stores them back.
#include "decode_common.hpp"
#include "fp8_append.hpp"

namespace pa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// KVNT: non-temporal K/V loads (large calls, as in the VALU kernel) or cacheable ones (calls of
// at most 256 MiB of KV, which fit the Infinity Cache: measured faster there, slower above)
template <int D, int BS, int NT, bool KV8, bool APPEND, bool KVNT>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeParams p) {
  constexpr int R = 16 * NT;         // query rows of one KV head handled by a workgroup
  constexpr int TPL = D / 32;        // consecutive V tokens a lane loads (one 8-dim chunk)
  constexpr int VTS = 20;            // V^T row stride in halves (16 tokens + 4): the staging
                                     // stores and the operand reads are both bank-conflict free
  constexpr int KK = D / 32;         // 32-dim steps of QK
  constexpr int MT = D / 16;         // 16-dim slices of the output
  constexpr int ESZ = KV8 ? 1 : 2;   // bytes per cached element
  constexpr int ROW_BYTES = D * ESZ;
  constexpr int TILE_BYTES = BS * ROW_BYTES;
  constexpr int LANE_BYTES = 8 * ESZ;  // 8 elements per lane per step
  constexpr int NWORDS = LANE_BYTES / 4;
  static_assert(BS % kRows == 0, "block size");

  const int hg = blockIdx.x;
  // grid row y decodes sequence seq_order[y] when the caller gives an order (clamped, so a bad
  // entry reads a wrong sequence, never outside the arrays)
  const int b = p.seq_order != nullptr ? min(max(p.seq_order[blockIdx.y], 0), (int)gridDim.y - 1)
                                       : (int)blockIdx.y;
  // partitions are dispatched last first: only long contexts have high partition indices, so
  // their full workgroups start early instead of forming the tail of the grid
  const int part = p.max_parts - 1 - (int)blockIdx.z;
  // query rows this workgroup owns: R, or fewer in a padded tile (the padding rows hold zero
  // queries and are never stored)
  const int rows = p.group / p.head_groups;
  const int kvh = hg / p.head_groups;
  const int h0 = kvh * p.group + (hg - kvh * p.head_groups) * rows;
  const SeqRange sr = seq_range<BS>(p, b);
  const int L = sr.L;
  const int part_tokens = p.part_tokens;
  const int span = L - sr.start;
  const int nparts = min(span > 0 ? (span + part_tokens - 1) / part_tokens : 1, p.max_parts);
  if (part >= nparts) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;  // K/V token row of a load; query row of a score
  const int lq = lane >> 4;  // 8-element group of a 32-dim step; 4-token group of a tile

  // ---- which 8 head dims lane (lr, lq) contributes to 32-dim step kk of QK ------------------
  // The contraction order is free, so it follows the loads: an fp16 lane loads 16 bytes (8 dims)
  // per step, dims 32 kk + 8 lq; an E4M3 lane loads 16 bytes (16 dims) for two steps at once,
  // dims 64 (kk / 2) + 16 lq + 8 (kk % 2), so that every K load instruction still covers 64
  // contiguous bytes of each of its 16 rows (8-byte loads would cover 32: as many memory
  // requests as for fp16, for half the bytes). q is gathered in the same order.
  constexpr int KL = KV8 ? KK / 2 : KK;  // 16-byte K loads per lane per tile
  auto kdim = [&](int kk) -> int {
    return KV8 ? 64 * (kk >> 1) + 16 * lq + 8 * (kk & 1) : 32 * kk + 8 * lq;
  };

  // ---- query rows as the B operand: row h0 + 16 nt + lr, dims kdim(kk) .. +8 ----------------
  h8 qb[NT][KK];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qb[nt][kk] = 16 * nt + lr < rows
                       ? *reinterpret_cast<const h8*>(p.q + ((size_t)b * p.num_q_heads + h0 +
                                                             16 * nt + lr) * D + kdim(kk))
                       : h8{0, 0, 0, 0, 0, 0, 0, 0};

  // ---- fused append: threads 0 .. 2 NEWC - 1 load the new K row's, then the new V row's
  // 16-byte chunks of fp16 (the rows exist for every sequence; the slot decides whether they
  // are used). s_new holds the rows as the cache stores them (fp16, or E4M3 codes under the
  // block's updated scale), then (E4M3) the scales before and after the append.
  constexpr int NEWC = D * 2 / 16;     // 16-byte fp16 chunks per new row
  constexpr int CODEB = ROW_BYTES / NEWC;  // cache bytes of one such chunk (16, or 8 for E4M3)
  __shared__ __align__(16) uint8_t s_new[APPEND ? 2 * ROW_BYTES + 16 : 16];
  Chunk<4> nrow{};
  int64_t new_slot = -1;
  int newtok = -1;  // position whose K/V come from s_new instead of the cache
  // E4M3: the last block's scales before (s_pk, s_pv) and after (s_k, s_v) the append, whether
  // its earlier codes are re-encoded (rk, rv), and its first position (last_start)
  float s_pk = 0.f, s_pv = 0.f, s_k = 1.f, s_v = 1.f;
  bool rk = false, rv = false;
  int last_start = 0x7fffffff;
  if constexpr (APPEND) {
    const size_t roff = (((size_t)b * p.num_kv_heads + kvh) * D + (tid % NEWC) * 8) * 2;
    if (tid < 2 * NEWC) nrow = load_chunk<4>((tid < NEWC ? p.k_new : p.v_new) + roff);
    new_slot = p.slot_mapping[b];
    if (new_slot >= 0 && new_slot < (int64_t)p.num_blocks * BS) newtok = L - 1;
    else new_slot = -1;  // skipped token, or a slot outside the pool: no append
    if (KV8 && newtok >= 0 && new_slot % BS > 0 && wave == 0) {
      const size_t si = (size_t)(new_slot / BS) * p.num_kv_heads + kvh;
      s_pk = p.k_scale[si];
      s_pv = p.v_scale[si];
    }
  }
  // the workgroup that stores the step's append: the first head group's last partition
  const bool appender = APPEND && new_slot >= 0 && (!KV8 || newtok >= 0) &&
                        hg == kvh * p.head_groups && part == nparts - 1;

  // ---- block ids of this wave's tokens: lane j holds logical block wbase / BS + j ------------
  // The partition's tokens [p0, p0 + pn) are split evenly over the waves in whole tiles, so a
  // short partition (the end of a context) keeps every wave busy. A full partition gives each
  // wave part_tokens / 4 tokens. p0 is a multiple of the block size and share of the tile, so a
  // tile never straddles a block of 16 tokens or more (and covers two whole blocks of 8), and
  // a wave's range spans at most 64 blocks.
  const int p0 = sr.start + part * part_tokens;
  const int pn = max(0, min(L - p0, part_tokens));
  const int share = (pn + kWaves * kTileTokens - 1) / (kWaves * kTileTokens) * kTileTokens;
  const int wbase = p0 + wave * share;
  const int woff = wbase % BS;  // lane j holds logical block wbase / BS + j
  const int nblk = min((L + BS - 1) / BS, p.max_blocks_per_seq);
  int my_id = 0;
  if (wbase < L) {
    const int lb = min(wbase / BS + lane, nblk - 1);
    my_id = p.block_tables[(size_t)b * p.max_blocks_per_seq + lb];
    my_id = min(max(my_id, 0), p.num_blocks - 1);
  }
  // E4M3: lane j also holds block j's K and V scales, loaded once with the ids (a scale load
  // inside the tile loop would put one more memory round trip into every tile)
  float my_ks = 1.f, my_vs = 1.f;
  if constexpr (KV8) {
    if (wbase < L) {
      my_ks = p.k_scale[(size_t)my_id * p.num_kv_heads + kvh];
      my_vs = p.v_scale[(size_t)my_id * p.num_kv_heads + kvh];
    }
  }
  // block of token (16 i + t) of tile i: uniform for BS >= 16; for BS = 8 the tile's second
  // half lies in the next block
  auto block_of = [&](int i, int t) -> int {
    const int j0 = (woff + kTileTokens * i) / BS;
    if constexpr (BS >= kTileTokens) {
      return __builtin_amdgcn_readlane(my_id, j0);
    } else {
      const int a = __builtin_amdgcn_readlane(my_id, j0);
      const int c = __builtin_amdgcn_readlane(my_id, j0 + 1);
      return t >= BS ? c : a;
    }
  };
  // the same lookup for a per-lane float (the block scales)
  auto lane_value_of = [&](float v, int i, int t) -> float {
    const int j0 = (woff + kTileTokens * i) / BS;
    const int vi = __builtin_bit_cast(int, v);
    if constexpr (BS >= kTileTokens) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, j0));
    } else {
      const int a = __builtin_amdgcn_readlane(vi, j0);
      const int c = __builtin_amdgcn_readlane(vi, j0 + 1);
      return __builtin_bit_cast(float, t >= BS ? c : a);
    }
  };

  const uint8_t* kbase = p.k_cache + (size_t)kvh * TILE_BYTES;
  const uint8_t* vbase = p.v_cache + (size_t)kvh * TILE_BYTES;
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE_BYTES;

  float m[NT], l[NT];
  f4 o[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = kNegInf;
    l[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nt][mt] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // LDS: a per-wave transposed V tile ([dim][token]), reused after the loop for the merge. The
  // merge area holds each wave's R x D partial with a row stride of D + 4 floats, so that the
  // 16 rows a wave writes with one instruction fall on different banks
  constexpr int DP = D + 4;
  constexpr int kMergeFloats = kWaves * R * (DP + 2);
  // fp16 caches: a per-wave K tile ([token][row bytes + 32]) as well; K is loaded in whole
  // rows and read back in the operand layout (see issue_tile)
  constexpr bool KROW = !KV8;
  constexpr int KRB = ROW_BYTES + 32;
  constexpr int kVtBytes = kWaves * D * VTS * 2;
  constexpr int kStageBytes = kVtBytes + (KROW ? kWaves * kTileTokens * KRB : 0);
  constexpr int kSmemFloats = kStageBytes > kMergeFloats * 4 ? kStageBytes / 4 : kMergeFloats;
  __shared__ __align__(16) float smem[kSmemFloats];
  _Float16* vt = reinterpret_cast<_Float16*>(smem) + wave * D * VTS;
  uint8_t* kt = reinterpret_cast<uint8_t*>(smem) + kVtBytes + wave * kTileTokens * KRB;

  // K is loaded in the MFMA operand layout; V as TPL consecutive tokens of one 8-dim chunk per
  // lane, so that it is stored transposed with one TPL-half store per dim
  const int vch = lane / (16 / TPL);   // 8-dim chunk
  const int vtg = lane % (16 / TPL);   // token group: tokens TPL vtg .. +TPL-1
  Chunk<4> ka[KL], kb[KL];
  // V loads. fp16: TPL consecutive tokens of one 8-dim chunk per lane (stored transposed). E4M3:
  // 16 bytes (16 dims) of one token row per lane, VLPR lanes per row and VRPI rows per load
  // instruction, so each instruction reads whole rows; they are stored as fp16 rows and the
  // P.V operand is read back with the transposed LDS read.
  constexpr int VLPR = ROW_BYTES / 16;
  constexpr int VRPI = 64 / VLPR;
  constexpr int VN = KV8 ? kTileTokens / VRPI : TPL;  // V loads per lane per tile
  constexpr int VRS = D + 16;                           // row stride (halves) of the E4M3 V tile
  static_assert(!KV8 || kTileTokens * VRS <= D * VTS, "row-major V tile fits the V^T tile");
  typedef Chunk<KV8 ? 4 : NWORDS> VChunk;
  VChunk va[VN], vb[VN];

  // K loads. fp16: LPR lanes cover one token row with 16 bytes each, RPI rows per instruction,
  // so every instruction reads whole rows, and consume_tile moves them to the operand layout
  // through LDS (loads straight into the operand layout read 64-byte row pieces per
  // instruction, which cost ~10 % of the HBM rate). E4M3: straight into the operand layout
  // (16 bytes per lane, two steps; the LDS round trip measured slower there).
  constexpr int LPR = ROW_BYTES / 16;
  constexpr int RPI = 64 / LPR;
  static_assert(!KROW || KL * RPI == kTileTokens, "K loads cover the tile");
  auto issue_tile = [&](int i, Chunk<4>(&kc)[KL], VChunk(&vc)[VN]) {
    if constexpr (KROW) {
#pragma unroll
      for (int c = 0; c < KL; ++c) {
        const int r = RPI * c + lane / LPR;
        const int id = block_of(i, r);
        const size_t off = (size_t)id * blk_stride +
                           (size_t)(((woff + kTileTokens * i + r) % BS) * ROW_BYTES) +
                           (size_t)(lane % LPR) * 16;
        kc[c] = load_chunk<4, KVNT>(kbase + off);
      }
    } else {
      const int id = block_of(i, lr);
      const size_t off =
          (size_t)id * blk_stride + (size_t)(((woff + kTileTokens * i + lr) % BS) * ROW_BYTES);
      // load c holds the dims of steps 2c and 2c + 1
#pragma unroll
      for (int c = 0; c < KL; ++c) kc[c] = load_chunk<4, KVNT>(kbase + off + kdim(2 * c));
    }
    if constexpr (KV8) {
#pragma unroll
      for (int c = 0; c < VN; ++c) {
        const int r = VRPI * c + lane / VLPR;
        const size_t voff = (size_t)block_of(i, r) * blk_stride +
                            (size_t)(((woff + kTileTokens * i + r) % BS) * ROW_BYTES) +
                            (size_t)(lane % VLPR) * 16;
        vc[c] = load_chunk<4, KVNT>(vbase + voff);
      }
    } else {
      // a lane's TPL tokens start at a multiple of TPL, so they share one block
      const int vid = block_of(i, TPL * vtg);
      const size_t voff = (size_t)vid * blk_stride +
                          (size_t)(((woff + kTileTokens * i + TPL * vtg) % BS) * ROW_BYTES +
                                   vch * LANE_BYTES);
#pragma unroll
      for (int u = 0; u < TPL; ++u)
        vc[u] = load_chunk<NWORDS, KVNT>(vbase + voff + (size_t)u * ROW_BYTES);
    }
  };

  // 8 elements of a chunk as fp16 (E4M3 codes decode exactly)
  auto to_h8 = [&](const Chunk<NWORDS>& c) -> h8 {
    uint32_t w[4];
    if constexpr (!KV8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = c.w[i];
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        w[2 * i] = e4m3x2_to_f16x2<false>(c.w[i]);
        w[2 * i + 1] = e4m3x2_to_f16x2<true>(c.w[i]);
      }
    }
    return __builtin_bit_cast(h8, w);
  };

  auto consume_tile = [&](int i, const Chunk<4>(&kc)[KL], const VChunk(&vc)[VN],
                          bool masked) {
    const int tok0 = wbase + kTileTokens * i;
    // per-token multipliers: softmax scale (and the K / V block scales of an E4M3 cache) for
    // this lane's four score tokens 4 lq + ii
    float kmul = p.scale_log2, vmul = 1.f;
    if constexpr (KV8) {
      // (E4M3 append: tokens of the last block use its updated scales; its tiles are masked)
      const bool last = APPEND && masked && tok0 + 4 * lq >= last_start;
      kmul *= last ? s_k : lane_value_of(my_ks, i, 4 * lq);
      vmul = last ? s_v : lane_value_of(my_vs, i, 4 * lq);
    }
    // chunk c of lane (lr, lq): token lr's dims of step c (fp16) or steps 2c and 2c + 1 (E4M3)
    Chunk<4> kcs[KL];
    if constexpr (KROW) {
#pragma unroll
      for (int c = 0; c < KL; ++c)
        store_chunk(kt + (RPI * c + lane / LPR) * KRB + (lane % LPR) * 16, kc[c]);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < KL; ++c) kcs[c] = load_chunk<4>(kt + lr * KRB + kdim(c) * ESZ);
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll
      for (int c = 0; c < KL; ++c) kcs[c] = kc[c];
    }
    if constexpr (APPEND && KV8) {
      // E4M3 append: the K codes of a token of the last block are re-encoded under its grown
      // scale, and stored back by the appending workgroup (positions before the new token);
      // the new token's codes come from s_new
      const int t = tok0 + lr;
      if (masked && rk && t >= last_start && t < newtok) {
        const int id = block_of(i, lr);
        const size_t off =
            (size_t)id * blk_stride + (size_t)(((woff + kTileTokens * i + lr) % BS) * ROW_BYTES);
#pragma unroll
        for (int c = 0; c < KL; ++c) {
#pragma unroll
          for (int w = 0; w < 4; ++w) kcs[c].w[w] = fp8_reencode_word(kcs[c].w[w], s_pk, s_k);
          if (appender)
            store_chunk(p.k_cache_w + (size_t)kvh * TILE_BYTES + off + kdim(2 * c), kcs[c]);
        }
      }
      if (masked && t == newtok) {
#pragma unroll
        for (int c = 0; c < KL; ++c) kcs[c] = load_chunk<4>(s_new + kdim(2 * c));
      }
    }
    h8 kA[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (KV8) {
        Chunk<NWORDS> half;  // the 8 codes of step kk
        half.w[0] = kcs[kk >> 1].w[2 * (kk & 1)];
        half.w[1] = kcs[kk >> 1].w[2 * (kk & 1) + 1];
        kA[kk] = to_h8(half);
      } else {
        kA[kk] = to_h8(kcs[kk]);
      }
    }
    if constexpr (APPEND && !KV8) {
      if (masked && tok0 + lr == newtok) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          kA[kk] = *reinterpret_cast<const h8*>(s_new + kdim(kk) * 2);
      }
    }
    h4 pB[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[kk], qb[nt][kk], s, 0, 0, 0);
      float sc[4];
      bool valid[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        valid[ii] = !masked || (tok0 + 4 * lq + ii < L);
        sc[ii] = valid[ii] ? mul_nc(s[ii], kmul) : kNegInf;
      }
      // online softmax for query row 16 nt + lr across the tile's 16 tokens
      float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      tm = fmaxf(tm, __shfl_xor(tm, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mn = fmaxf(m[nt], tm);
      const float ms = mn == kNegInf ? 0.f : mn;
      const float alpha = fexp2(m[nt] - ms);
      float pw[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) pw[ii] = fexp2(sc[ii] - ms);
      l[nt] = l[nt] * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
      m[nt] = mn;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
      pB[nt] = h4{(_Float16)(pw[0] * vmul), (_Float16)(pw[1] * vmul), (_Float16)(pw[2] * vmul),
                  (_Float16)(pw[3] * vmul)};
    }
    if constexpr (KV8) {
      // E4M3: each lane's 16 codes of row r (token tok0 + r), converted, into the wave's
      // row-major fp16 V tile; tokens past the context are zeros so that stale or poisoned
      // slots cannot reach the sums
#pragma unroll
      for (int c = 0; c < VN; ++c) {
        const int r = VRPI * c + lane / VLPR;
        const int q = lane % VLPR;
        const int t = tok0 + r;
        Chunk<4> vcs = vc[c];
        if constexpr (APPEND) {
          if (masked && rv && t >= last_start && t < newtok) {
#pragma unroll
            for (int w = 0; w < 4; ++w) vcs.w[w] = fp8_reencode_word(vcs.w[w], s_pv, s_v);
            if (appender) {
              const size_t voff = (size_t)block_of(i, r) * blk_stride +
                                  (size_t)(((woff + kTileTokens * i + r) % BS) * ROW_BYTES);
              store_chunk(p.v_cache_w + (size_t)kvh * TILE_BYTES + voff + (size_t)q * 16, vcs);
            }
          }
          if (masked && t == newtok) vcs = load_chunk<4>(s_new + ROW_BYTES + q * 16);
        }
        Chunk<NWORDS> lo, hi;
        lo.w[0] = vcs.w[0];
        lo.w[1] = vcs.w[1];
        hi.w[0] = vcs.w[2];
        hi.w[1] = vcs.w[3];
        h8 vlo = to_h8(lo), vhi = to_h8(hi);
        if (masked && t >= L) vlo = vhi = h8{0, 0, 0, 0, 0, 0, 0, 0};
        *reinterpret_cast<h8*>(vt + r * VRS + 16 * q) = vlo;
        *reinterpret_cast<h8*>(vt + r * VRS + 16 * q + 8) = vhi;
      }
      __builtin_amdgcn_wave_barrier();
      // O^T += V^T P^T; the A operand (dim 16 mt + lr, tokens 4 lq .. +3) comes out of the
      // row-major tile with gfx950's transposed read: within each 16-lane group, lane lr passes
      // 4 halves of the row of token 4 lq + lr / 4 and receives, as element e, half lr % 4 of
      // the row passed by lane 4 e + lr / 4
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        typedef short s4 __attribute__((ext_vector_type(4)));
        const s4 rd = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(
            vt + (4 * lq + (lr >> 2)) * VRS + 16 * mt + 4 * (lr & 3)));
        const h4 vA = __builtin_bit_cast(h4, rd);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vA, pB[nt], o[nt][mt], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      // stage V transposed as fp16: dim 8 vch + e gets this lane's TPL tokens in one store;
      // tokens past the context are zeros so that stale or poisoned slots cannot reach the sums
      h8 vv[TPL];
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        vv[u] = to_h8(vc[u]);
        if constexpr (APPEND) {
          if (masked && tok0 + TPL * vtg + u == newtok)
            vv[u] = *reinterpret_cast<const h8*>(s_new + ROW_BYTES + vch * 16);
        }
        if (masked && tok0 + TPL * vtg + u >= L) vv[u] = h8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16* dst = vt + (8 * vch + e) * VTS + TPL * vtg;
        if constexpr (TPL == 4)
          *reinterpret_cast<h4*>(dst) = h4{vv[0][e], vv[1][e], vv[2][e], vv[3][e]};
        else
          *reinterpret_cast<h2v*>(dst) = h2v{vv[0][e], vv[1][e]};
      }
      __builtin_amdgcn_wave_barrier();
      // O^T[dim][row] += V^T[dim][token] P^T[token][row], 16 dims at a time; the A operand (dim
      // 16 mt + lr, tokens 4 lq .. +3) is one 8-byte read
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const h4 vA = *reinterpret_cast<const h4*>(vt + (16 * mt + lr) * VTS + 4 * lq);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(vA, pB[nt], o[nt][mt], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    }
  };

  // same double-buffered walk as the VALU kernel (unconditional loads in the steady state)
  const int avail = max(0, min(p0 + pn - wbase, share));
  int n_full = avail / kTileTokens;
  bool has_tail = (avail % kTileTokens) != 0;
  if constexpr (APPEND) {
    // the new token is the wave's last attended position: its tile takes the masked path
    if (!has_tail && n_full > 0 && newtok >= wbase && newtok < wbase + avail) {
      --n_full;
      has_tail = true;
    }
  }
  const int n_tiles = n_full + (has_tail ? 1 : 0);
  if (n_tiles > 0) issue_tile(0, ka, va);
  if constexpr (APPEND && !KV8) {
    // after the first tile's loads: the block-id wait before them has already retired the
    // new-row loads, so staging them costs no extra round trip
    if (tid < 2 * NEWC)
      *reinterpret_cast<u32x4*>(s_new + tid * 16) = u32x4{nrow.w[0], nrow.w[1], nrow.w[2], nrow.w[3]};
    __syncthreads();
  }
  if constexpr (APPEND && KV8) {
    // wave 0 applies the block-scale policy to the new rows: row maxima over the NEWC lanes of
    // each row (one DPP row or half-row), the scales, and the codes under them
    if (wave == 0 && newtok >= 0) {
      float x[8], a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (float)__builtin_bit_cast(h2v, nrow.w[e / 2])[e % 2];
        a = fmaxf(a, fabsf(x[e]));
      }
      a = lane_group_max<NEWC>(a);
      const float sk = uniform(fp8_append_scale(a, s_pk));
      const float sv = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fp8_append_scale(a, s_pv)), NEWC));
      const float s = tid < NEWC ? sk : sv;
      u32x2 c;
#pragma unroll
      for (int w = 0; w < 2; ++w)
        c[w] = enc_pair<true>(x[4 * w + 2] / s, x[4 * w + 3] / s,
                              enc_pair<false>(x[4 * w] / s, x[4 * w + 1] / s, 0u));
      if (tid < 2 * NEWC)
        *reinterpret_cast<u32x2*>(s_new + (tid < NEWC ? 0 : ROW_BYTES) + (tid % NEWC) * CODEB) = c;
      if (tid == 0)
        *reinterpret_cast<f4*>(s_new + 2 * ROW_BYTES) = f4{s_pk, sk, s_pv, sv};
    }
    __syncthreads();
  }
  if constexpr (APPEND && KV8) {
    if (newtok >= 0) {
      const f4 sc = *reinterpret_cast<const f4*>(s_new + 2 * ROW_BYTES);
      const int off = (int)(new_slot % BS);
      s_pk = uniform(sc[0]);
      s_k = uniform(sc[1]);
      s_pv = uniform(sc[2]);
      s_v = uniform(sc[3]);
      rk = s_k != s_pk && off > 0;
      rv = s_v != s_pv && off > 0;
      last_start = newtok - off;
    }
  }

  int i = 0;
  if constexpr (APPEND && KV8) {
    // E4M3 append: every tile holding a position of the last block takes the masked path
    const int first_masked = max(0, (last_start - wbase) / kTileTokens);
    for (; i + 2 < n_tiles && i + 2 <= first_masked; i += 2) {
      issue_tile(i + 1, kb, vb);
      consume_tile(i, ka, va, false);
      issue_tile(i + 2, ka, va);
      consume_tile(i + 1, kb, vb, false);
    }
    const bool last_has_tail = has_tail;
    auto masked_at = [&](int t) {
      return t >= first_masked || (t == n_tiles - 1 && last_has_tail);
    };
    for (; i + 2 < n_tiles; i += 2) {
      issue_tile(i + 1, kb, vb);
      consume_tile(i, ka, va, masked_at(i));
      issue_tile(i + 2, ka, va);
      consume_tile(i + 1, kb, vb, masked_at(i + 1));
    }
    if (i + 1 < n_tiles) {
      issue_tile(i + 1, kb, vb);
      consume_tile(i, ka, va, masked_at(i));
      consume_tile(i + 1, kb, vb, masked_at(i + 1));
    } else if (i < n_tiles) {
      consume_tile(i, ka, va, masked_at(i));
    }
  } else {
    for (; i + 2 < n_tiles; i += 2) {
      issue_tile(i + 1, kb, vb);
      consume_tile(i, ka, va, false);
      issue_tile(i + 2, ka, va);
      consume_tile(i + 1, kb, vb, false);
    }
    if (i + 1 < n_tiles) {
      issue_tile(i + 1, kb, vb);
      consume_tile(i, ka, va, false);
      consume_tile(i + 1, kb, vb, has_tail);
    } else if (i < n_tiles) {
      consume_tile(i, ka, va, has_tail);
    }
  }

  // fused append: the first head group's last partition stores the new rows at their slot
  // (E4M3: and the block's scales)
  if constexpr (APPEND) {
    if (appender && tid < 2 * NEWC) {
      const int64_t blk = new_slot / BS;
      const int off = (int)(new_slot - blk * BS);
      const size_t dst = ((size_t)blk * p.num_kv_heads + kvh) * TILE_BYTES +
                         (size_t)off * ROW_BYTES + (size_t)(tid % NEWC) * CODEB;
      uint8_t* cache = tid < NEWC ? p.k_cache_w : p.v_cache_w;
      const uint8_t* src = s_new + (tid < NEWC ? 0 : ROW_BYTES) + (tid % NEWC) * CODEB;
      if constexpr (KV8) {
        *reinterpret_cast<u32x2*>(cache + dst) = *reinterpret_cast<const u32x2*>(src);
        if (tid == 0) {
          p.k_scale_w[(size_t)blk * p.num_kv_heads + kvh] = s_k;
          p.v_scale_w[(size_t)blk * p.num_kv_heads + kvh] = s_v;
        }
      } else {
        *reinterpret_cast<u32x4*>(cache + dst) = *reinterpret_cast<const u32x4*>(src);
      }
    }
  }

  // row sums: the four lanes of a row held partial sums over their own tokens
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    l[nt] += __shfl_xor(l[nt], 16);
    l[nt] += __shfl_xor(l[nt], 32);
  }

  // ---- merge the kWaves waves through LDS (the staging area is reused) ----------------------
  __syncthreads();
  float* s_acc = smem;                              // [kWaves][R][DP]
  float* s_ml = smem + kWaves * R * DP;             // [kWaves][R][2]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = 16 * nt + lr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f4*>(s_acc + (wave * R + row) * DP + 16 * mt + 4 * lq) = o[nt][mt];
    if (lq == 0) {
      s_ml[(wave * R + row) * 2] = m[nt];
      s_ml[(wave * R + row) * 2 + 1] = l[nt];
    }
  }
  __syncthreads();

  // Each row's running max, wave weights and running sum are formed once (one thread per row)
  // and then shared by its D elements, in the order a per-element merge would use.
  __shared__ float s_wt[kWaves][R];
  __shared__ float s_row[R][2];
  if (tid < rows) {
    const int h = tid;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_ml[(w * R + h) * 2]);
    const float ms = mx == kNegInf ? 0.f : mx;
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fexp2(s_ml[(w * R + h) * 2] - ms);
      ls = fmaf(wt, s_ml[(w * R + h) * 2 + 1], ls);
      s_wt[w][h] = wt;
    }
    s_row[h][0] = mx;
    s_row[h][1] = ls;
  }
  __syncthreads();

  // dims d0 .. d0 + 3 of row h: one 16-byte LDS read per wave
  auto local_merge = [&](int h, int d0, float& mx, float& ls, float (&a)[4]) {
    mx = s_row[h][0];
    ls = s_row[h][1];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = s_wt[w][h];
      const f4 x = *reinterpret_cast<const f4*>(s_acc + (w * R + h) * DP + d0);
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = fmaf(wt, x[u], a[u]);
    }
  };
  finish_partition<R, D, kThreads, 4>(p, b, hg, part, nparts, sr.extra, h0, rows, local_merge);
}

template <int D, int BS, int NT, bool KV8, bool APPEND>
hipError_t launch_one(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads * p.head_groups, num_seqs, p.max_parts);
  if (p.kv_cached)
    decode_mfma_kernel<D, BS, NT, KV8, APPEND, false><<<grid, kThreads, 0, stream>>>(p);
  else
    decode_mfma_kernel<D, BS, NT, KV8, APPEND, true><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, bool KV8, int NT, bool APPEND>
hipError_t dispatch_bs(const DecodeParams& p, int num_seqs, int bs, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_one<D, 8, NT, KV8, APPEND>(p, num_seqs, stream);
    case 16: return launch_one<D, 16, NT, KV8, APPEND>(p, num_seqs, stream);
    case 32: return launch_one<D, 32, NT, KV8, APPEND>(p, num_seqs, stream);
    case 64: return launch_one<D, 64, NT, KV8, APPEND>(p, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool KV8, bool APPEND = false>
hipError_t dispatch_rows(const DecodeParams& p, int num_seqs, int bs, int rows, hipStream_t stream) {
  return rows > 16 ? dispatch_bs<D, KV8, 2, APPEND>(p, num_seqs, bs, stream)
                    : dispatch_bs<D, KV8, 1, APPEND>(p, num_seqs, bs, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                              int rows, bool kv_fp8, hipStream_t stream) {
  if (head_dim == 128)
    return kv_fp8 ? dispatch_rows<128, true>(p, num_seqs, block_size, rows, stream)
                  : dispatch_rows<128, false>(p, num_seqs, block_size, rows, stream);
  if (head_dim == 64)
    return kv_fp8 ? dispatch_rows<64, true>(p, num_seqs, block_size, rows, stream)
                  : dispatch_rows<64, false>(p, num_seqs, block_size, rows, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma_append(const DecodeParams& p, int num_seqs, int head_dim,
                                     int block_size, int rows, bool kv_fp8, hipStream_t stream) {
  if (head_dim == 128)
    return kv_fp8 ? dispatch_rows<128, true, true>(p, num_seqs, block_size, rows, stream)
                  : dispatch_rows<128, false, true>(p, num_seqs, block_size, rows, stream);
  if (head_dim == 64)
    return kv_fp8 ? dispatch_rows<64, true, true>(p, num_seqs, block_size, rows, stream)
                  : dispatch_rows<64, false, true>(p, num_seqs, block_size, rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

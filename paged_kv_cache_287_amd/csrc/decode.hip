// Paged decode attention for gfx950 (CDNA4): split-context partition kernel + exact merge.
//
// What is computed (per sequence b, query head h, KV head g = h / G):
//   out[b, h] = softmax(scale * K_b q) V_b, where token t of K_b / V_b lives in physical block
//   block_tables[b, t / BS] at offset t % BS ("serving-paged-attention", section "블록으로
//   쪼개고 표로 잇는다": attention looks the scattered blocks up through the table). The softmax
//   is evaluated online, tile by tile, tracking a running maximum, a running sum of
//   exponentials and a running weighted value sum, so no score matrix ever leaves the chip
//   (talk summary, FlashAttention paragraph: tiles kept on chip, three running quantities).
//   Decode reads every cached byte once per step and is bound by memory bandwidth (talk
//   summary, prefill/decode paragraphs), so the kernel is organised around HBM traffic.
//
// Mapping onto CDNA4:
//   * workgroup = (KV head [x GT query heads], sequence, context partition), 4 waves; the
//     partition's tokens are split evenly over the waves in whole tiles of a few steps.
//   * within a wave, LPT consecutive lanes hold one token per step, each lane 16 contiguous
//     bytes of it (8 for E4M3 rows of 64 elements in blocks of 8): LPT = 16 for fp16 rows of 128
//     elements, 8 for E4M3 rows of 128 or fp16 rows of 64, 4 for E4M3 rows of 64. One step of
//     the wave therefore loads 64 / LPT consecutive token rows of a block, 1 KiB of contiguous
//     memory. K and V use the same addressing.
//   * q . k: v_dot2 (fp16 x fp16 -> fp32) over the lane's elements, then an all-reduce over the
//     token's lanes with DPP adds (quad_perm xor 1, xor 2, row_half_mirror, row_mirror). Every
//     lane of the token ends with the bit-identical score.
//   * each token row keeps its own online-softmax state (max, sum) per query head and a partial
//     output of E floats per lane and head; the rows of a 16-lane DPP row merge in registers,
//     then DPP rows and waves once, through LDS, at the end of the partition. Scores are kept in
//     log2 units (scale * log2 e folded in) so the exponentials are single v_exp_f32
//     instructions. The running maximum only moves when a score passes it by more than 8 (log2
//     units), which skips the rescaling of most tiles.
//   * P.V: a lane's tokens of two steps are paired element by element, so one v_dot2 per
//     element and head adds two tokens' contributions (probabilities rounded to fp16).
//   * the block ids a wave needs are fetched once, one per lane, and read back with
//     v_readlane, so the table walk costs no memory latency inside the tile loop; the next
//     tile's K and V loads are issued before the current tile is consumed.
//   * grid x = head group x KV heads + KV head is the fastest-varying dimension; with a multiple
//     of 8 KV heads the round-robin dispatch of workgroups over the 8 XCDs puts every workgroup
//     of one KV head on one XCD, so blocks shared by several head groups or sequences (a common
//     prefix) are re-read from that XCD's L2.
//   * results depend only on logical token positions (fixed tile, row and merge order), so
//     they are deterministic and independent of physical block placement.
//   * fused append (APPEND): the step's new token of each sequence (position L - 1, K/V rows
//     given beside the cache) is both stored at its slot and attended in the same launch. Every
//     workgroup that covers position L - 1 takes that token's K/V from the new rows instead of
//     the cache, so no workgroup depends on another's store; the first head group of each KV
//     head stores the rows from its last partition. The result is bit-identical to appending
//     first and decoding afterwards. With an 8-bit cache (one head group per KV head, so one
//     workgroup reads the last block) that workgroup also applies the block-scale policy: the
//     new rows are encoded under the updated scale, and when the scale grows the block's
//     earlier codes are re-encoded as they are read (the tiles of the last block take the
//     masked path) and stored back with the new scales.
#include "decode_common.hpp"
#include "fp8_append.hpp"
#include "prefill_body.hpp"

namespace pa {
namespace {

// Sum over groups of LPT consecutive lanes (4, 8 or 16) of a DPP row; every lane of a group
// receives the same bits.
template <int LPT>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "lane group");
  x += dpp_mov<0xB1>(x);                          // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);                          // quad_perm [2,3,0,1]
  if constexpr (LPT >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: pairs the quads of a half-row
  if constexpr (LPT >= 16) x += dpp_mov<0x140>(x); // row_mirror: pairs the two half-rows
  return x;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                c, false);
}


// Per-lane view of one token's elements as fp16 pairs (E/2 words).
template <int E, bool KV8>
__device__ __forceinline__ void to_half_pairs(const Chunk<(KV8 ? E : 2 * E) / 4>& c,
                                              uint32_t (&h)[E / 2]) {
  if constexpr (!KV8) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) h[i] = c.w[i];
  } else {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      h[2 * i] = e4m3x2_to_f16x2<false>(c.w[i]);
      h[2 * i + 1] = e4m3x2_to_f16x2<true>(c.w[i]);
    }
  }
}

// Largest step of a row's score above the running-max reference before l and acc are
// rescaled (log2 units): probabilities stay below 256.
constexpr float kRescaleSlack = 8.f;

// Lane layout of one token's row of D cached elements: LPT consecutive lanes hold it, each
// LANE_BYTES contiguous bytes (16 wherever the row allows it, so every lane issues one 16-byte
// load), and one wave step covers RW = 64 / LPT consecutive tokens of one block. A tile is NSTEP
// steps, two where a lane's partial outputs (E per query head) already take 64 registers.
// Fewer lanes per token means fewer per-token instructions (score reduction, softmax) per byte,
// which is what bounds the kernel when 8-bit codes halve the bytes per token.
template <int D, int BS, int GT, bool KV8>
struct RowLayout {
  static constexpr int ESZ = KV8 ? 1 : 2;                       // bytes per cached element
  static constexpr int ROW_BYTES = D * ESZ;                     // one token of one head
  static constexpr int LPT = ROW_BYTES / 16 > kWave / BS ? ROW_BYTES / 16 : kWave / BS;
  static constexpr int LANE_BYTES = ROW_BYTES / LPT;            // 16, or 8 for E4M3 D 64 BS 8
  static constexpr int E = D / LPT;                             // elements per lane per token
  static constexpr int RW = kWave / LPT;                        // tokens per wave step
  static constexpr int NSTEP = E * GT >= 64 ? 2 : 4;            // steps per tile
  static constexpr int TT = RW * NSTEP;                         // tokens per tile
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "lane groups are 4, 8 or 16 lanes");
  static_assert(BS % RW == 0, "a step's tokens share a block");
  static_assert(NSTEP % 2 == 0, "P.V pairs the tokens of two steps");
};

// Merge the online-softmax state of this lane with that of the lane CTRL (a DPP row rotation)
// points to; both hold the same elements of different tokens.
template <int CTRL, int GT, int E>
__device__ __forceinline__ void merge_lane_states(float (&m)[GT], float (&l)[GT],
                                                  float (&acc)[GT][E]) {
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const float mo = dpp_mov<CTRL>(m[h]);
    const float lo = dpp_mov<CTRL>(l[h]);
    const float mn = fmaxf(m[h], mo);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float a = fexp2(m[h] - ms);
    const float c = fexp2(mo - ms);
    l[h] = a * l[h] + c * lo;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = a * acc[h][e] + c * dpp_mov<CTRL>(acc[h][e]);
    m[h] = mn;
  }
}

// LDS of one decode workgroup: the partial state of its 16 DPP rows (4 per wave) for the merge.
template <int D, int GT>
constexpr size_t decode_lds_bytes() {
  return (size_t)kWaves * (kWave / 16) * GT * (D + 2) * sizeof(float);
}

// One (head group hg, grid row y, partition) workgroup of a grid with nseq rows. KV_NT: the K/V
// tiles are read with non-temporal loads (streamed past the caches: every byte is read once per
// call); without it they may stay in L2 for other workgroups of the same KV head on that XCD
// (shared-prefix batches, whose forked siblings also share their tails).
template <int D, int BS, int GT, bool KV8, bool APPEND, bool KV_NT = true>
__device__ __forceinline__ void decode_body(const DecodeParams& p, int hg, int y, int part_idx,
                                            int nseq, uint8_t* lds) {
  using Lay = RowLayout<D, BS, GT, KV8>;
  constexpr int LPT = Lay::LPT;
  constexpr int E = Lay::E;
  constexpr int RW = Lay::RW;
  constexpr int NSTEP = Lay::NSTEP;
  constexpr int TT = Lay::TT;
  constexpr int LANE_BYTES = Lay::LANE_BYTES;
  constexpr int NWORDS = LANE_BYTES / 4;
  constexpr int NH2 = E / 2;                // fp16 pairs per lane per token
  constexpr int ROW_BYTES = Lay::ROW_BYTES;
  constexpr int TILE_BYTES = BS * ROW_BYTES;  // one (block, head) tile
  // host-validated: part_tokens is a power of two in [256, 4096] with part_tokens / 4 <= 64 * BS,
  // so a wave's tokens are whole blocks and fit one block id per lane

  // With 8 or more KV heads, head groups of one KV head are kvh, kvh + Hkv, ...: workgroup ids
  // are dealt round-robin over the 8 XCDs, so all of them read that KV head through one L2.
  // grid row y decodes sequence seq_order[y] when the caller gives an order (clamped, so a bad
  // entry reads a wrong sequence, never outside the arrays)
  const int b = p.seq_order != nullptr ? min(max(p.seq_order[y], 0), nseq - 1) : y;
  // Dispatch order of the partitions (grid z). In batch order, partition 0 of every sequence
  // goes first: that is the full-size piece of every long context, while higher indices exist
  // only for long contexts and end with their partial last piece; the reverse left full pieces
  // for the end of the grid (uneven lengths at 128 x [32, 8192] tokens: 153 -> 148.5 us). With
  // a caller's longest-first order the last partitions go first instead: the grid then ends
  // with partition 0 of the shortest contexts, the smallest pieces of all (same lengths: 145 ->
  // 138 us).
  const int part = p.seq_order != nullptr ? p.max_parts - 1 - part_idx : part_idx;
  const int kvh = hg % p.num_kv_heads;
  const int h0 = kvh * p.group + (hg / p.num_kv_heads) * GT;
  const SeqRange sr = seq_range<BS>(p, b);
  const int L = sr.L;
  // partitions beyond the grid's (context longer than the host bound) are dropped, never
  // written outside the workspace
  const int part_tokens = p.part_tokens;
  const int span = L - sr.start;
  const int nparts = min(span > 0 ? (span + part_tokens - 1) / part_tokens : 1, p.max_parts);
  if (part >= nparts) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = lane / LPT;   // token of the step
  const int col = lane % LPT;   // element chunk [col * E, col * E + E)

  // ---- fused append: this lane's chunk of the new token's K and V rows ------------------
  // Loaded whether or not the sequence appends (the row exists for every sequence), so the
  // loads do not wait for the slot; newtok = L - 1 marks the position taken from them.
  Chunk<NWORDS> knew{}, vnew{};
  int64_t new_slot = -1;
  int newtok = -1;
  // E4M3: the last block's scales before (s_pk, s_pv) and after (s_k, s_v) the append, whether
  // its earlier codes are re-encoded (rk, rv), and its first position (last_start)
  float s_pk = 0.f, s_pv = 0.f, s_k = 1.f, s_v = 1.f;
  bool rk = false, rv = false;
  int last_start = 0x7fffffff;
  if constexpr (APPEND && !KV8) {
    const size_t nrow = ((size_t)b * p.num_kv_heads + kvh) * ROW_BYTES + col * LANE_BYTES;
    knew = load_chunk<NWORDS>(p.k_new + nrow);
    vnew = load_chunk<NWORDS>(p.v_new + nrow);
    new_slot = p.slot_mapping[b];
    if (new_slot >= 0 && new_slot < (int64_t)p.num_blocks * BS) newtok = L - 1;
    else new_slot = -1;  // skipped token, or a slot outside the pool: no append
  }
  if constexpr (APPEND && KV8) {
    // the lane's E fp16 elements of the new rows (E = 4 * NWORDS, 2E bytes)
    constexpr int NC = E / 8;  // 16-byte chunks
    const size_t nrow = (((size_t)b * p.num_kv_heads + kvh) * D + col * E) * 2;
    Chunk<4> kx[NC], vx[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kx[c] = load_chunk<4>(p.k_new + nrow + 16 * c);
      vx[c] = load_chunk<4>(p.v_new + nrow + 16 * c);
    }
    new_slot = p.slot_mapping[b];
    if (new_slot >= 0 && new_slot < (int64_t)p.num_blocks * BS) newtok = L - 1;
    else new_slot = -1;
    if (newtok >= 0) {
      const int64_t blk = new_slot / BS;
      const int off = (int)(new_slot - blk * BS);
      last_start = newtok - off;
      if (off > 0) {
        s_pk = p.k_scale[(size_t)blk * p.num_kv_heads + kvh];
        s_pv = p.v_scale[(size_t)blk * p.num_kv_heads + kvh];
      }
      float xk[E], xv[E];
      float ak = 0.f, av = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t wk = kx[e / 8].w[(e % 8) / 2], wv = vx[e / 8].w[(e % 8) / 2];
        xk[e] = (float)__builtin_bit_cast(half2_t, wk)[e % 2];
        xv[e] = (float)__builtin_bit_cast(half2_t, wv)[e % 2];
        ak = fmaxf(ak, fabsf(xk[e]));
        av = fmaxf(av, fabsf(xv[e]));
      }
      // every lane group holds the whole row, so the row maximum is wave-uniform
      s_k = uniform(fp8_append_scale(lane_group_max<LPT>(ak), s_pk));
      s_v = uniform(fp8_append_scale(lane_group_max<LPT>(av), s_pv));
      rk = s_k != s_pk && off > 0;
      rv = s_v != s_pv && off > 0;
#pragma unroll
      for (int w = 0; w < NWORDS; ++w) {
        knew.w[w] = enc_pair<true>(xk[4 * w + 2] / s_k, xk[4 * w + 3] / s_k,
                                   enc_pair<false>(xk[4 * w] / s_k, xk[4 * w + 1] / s_k, 0u));
        vnew.w[w] = enc_pair<true>(xv[4 * w + 2] / s_v, xv[4 * w + 3] / s_v,
                                   enc_pair<false>(xv[4 * w] / s_v, xv[4 * w + 1] / s_v, 0u));
      }
    }
  }
  // the workgroup that stores the step's append: the first head group's last partition
  const bool appender = APPEND && new_slot >= 0 && (!KV8 || newtok >= 0) && hg < p.num_kv_heads &&
                        part == nparts - 1;

  // ---- query rows of this head group: E fp16 per lane per head -------------------------
  uint32_t qw[GT][NH2];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(
        p.q + ((size_t)b * p.num_q_heads + h0 + h) * D + col * E);
#pragma unroll
    for (int c = 0; c < NH2 / 4; ++c) {
      const Chunk<4> ch = load_chunk<4>(qp + 16 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) qw[h][4 * c + i] = ch.w[i];
    }
  }

  // ---- block ids of this wave's tokens: lane j holds logical block lb0 + j ---------------
  // The partition's tokens [p0, p0 + pn) are split evenly over the waves in whole tiles, so a
  // short partition (the end of a context) keeps every wave busy. A full partition gives each
  // wave part_tokens / 4 tokens. p0 is a multiple of the block size and share of the tile, so a
  // step never straddles a block, and a wave's range spans at most 64 blocks.
  const int p0 = sr.start + part * part_tokens;
  const int pn = max(0, min(L - p0, part_tokens));
  const int share = (pn + kWaves * TT - 1) / (kWaves * TT) * TT;
  const int wbase = p0 + wave * share;
  const int woff = wbase % BS;  // lane j holds logical block wbase / BS + j
  const int nblk = min((L + BS - 1) / BS, p.max_blocks_per_seq);
  int my_id = 0;
  if (wbase < L) {
    const int lb = min(wbase / BS + lane, nblk - 1);
    my_id = p.block_tables[(size_t)b * p.max_blocks_per_seq + lb];
    my_id = min(max(my_id, 0), p.num_blocks - 1);  // a bad id reads a wrong block, never outside the pool
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

  const uint8_t* kbase = p.k_cache + (size_t)kvh * TILE_BYTES;
  const uint8_t* vbase = p.v_cache + (size_t)kvh * TILE_BYTES;
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE_BYTES;
  const int lane_off = row * ROW_BYTES + col * LANE_BYTES;

  float m[GT], l[GT], acc[GT][E];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  Chunk<NWORDS> ka[NSTEP], va[NSTEP], kb[NSTEP], vb[NSTEP];

  auto issue_tile = [&](int i, Chunk<NWORDS>(&kc)[NSTEP], Chunk<NWORDS>(&vc)[NSTEP]) {
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const int t = TT * i + RW * s;  // first token of the step, wave-relative
      const int id = __builtin_amdgcn_readlane(my_id, (woff + t) / BS);
      const size_t off = (size_t)id * blk_stride + (size_t)(((woff + t) % BS) * ROW_BYTES + lane_off);
      kc[s] = load_chunk<NWORDS, KV_NT>(kbase + off);
      vc[s] = load_chunk<NWORDS, KV_NT>(vbase + off);
    }
  };

  // E4M3 append: a step of the last block whose scale grew re-encodes its codes; the appending
  // workgroup stores them back (positions before the new token: the new row is stored once
  // below). Every lane writes only the bytes it loaded, and no other workgroup reads the block.
  auto fix_step = [&](Chunk<NWORDS>& c, int t, float s_prev, float s_new, uint8_t* cache_w) {
    Chunk<NWORDS> r;
#pragma unroll
    for (int w = 0; w < NWORDS; ++w) r.w[w] = fp8_reencode_word(c.w[w], s_prev, s_new);
    c = r;
    if (appender && wbase + t + row < newtok) {
      const int id = __builtin_amdgcn_readlane(my_id, (woff + t) / BS);
      const size_t off = (size_t)kvh * TILE_BYTES + (size_t)id * blk_stride +
                         (size_t)(((woff + t) % BS) * ROW_BYTES + lane_off);
      store_chunk(cache_w + off, r);
    }
  };

  auto consume_tile = [&](int i, const Chunk<NWORDS>(&kc)[NSTEP],
                          const Chunk<NWORDS>(&vc)[NSTEP], bool masked) {
    const int tok0 = wbase + TT * i;
    float sc[NSTEP][GT];
    float kmul[NSTEP], vmul[NSTEP];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      kmul[s] = p.scale_log2;
      vmul[s] = 1.f;
      // (wave-uniform; the tiles holding the last block are consumed as masked tiles)
      const bool in_last = APPEND && KV8 && masked && tok0 + RW * s >= last_start;
      if constexpr (KV8) {
        const int t = TT * i + RW * s;
        const int j = (woff + t) / BS;
        kmul[s] *= in_last ? s_k : __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_ks), j));
        vmul[s] = in_last ? s_v : __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_vs), j));
      }
      uint32_t kh[NH2];
      Chunk<NWORDS> kcs = kc[s];
      if constexpr (APPEND && KV8) {
        if (in_last && rk) fix_step(kcs, TT * i + RW * s, s_pk, s_k, p.k_cache_w);
      }
      if constexpr (APPEND) {
        if (masked && tok0 + RW * s + row == newtok) kcs = knew;
      }
      to_half_pairs<E, KV8>(kcs, kh);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float d = 0.f;
#pragma unroll
        for (int w = 0; w < NH2; ++w) d = dot2(kh[w], qw[h][w], d);
        sc[s][h] = d;
      }
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const bool valid = !masked || (tok0 + RW * s + row < L);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float x = mul_nc(lane_group_sum<LPT>(sc[s][h]), kmul[s]);
        sc[s][h] = valid ? x : kNegInf;
      }
    }
    // Online softmax. The running maximum m is only the reference point of l and acc (both are
    // sums of 2^(s - m) terms), so it moves, and l and acc are rescaled, only when some row's
    // score exceeds it by more than kRescaleSlack; probabilities then stay below 2^kRescaleSlack.
    // The decision is wave-uniform and the result is the same softmax up to rounding.
    float pw[NSTEP][GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int s = 1; s < NSTEP; ++s) mt = fmaxf(mt, sc[s][h]);
      if (__builtin_amdgcn_ballot_w64(mt > m[h] + kRescaleSlack) != 0) {
        const float mn = fmaxf(m[h], mt);
        const float alpha = fexp2(m[h] - (mn == kNegInf ? 0.f : mn));
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
      const float ms = m[h] == kNegInf ? 0.f : m[h];
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) pw[s][h] = fexp2(sc[s][h] - ms);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < NSTEP / 2; ++j) ps += pw[2 * j][h] + pw[2 * j + 1][h];
      l[h] += ps;
    }
    // Weighted value sum as fp16 dot products over token pairs: the lane's tokens of steps 2j
    // and 2j + 1 are paired element by element (byte permutes), the two probabilities rounded
    // to fp16, and one v_dot2 per element and head adds both tokens.
    uint32_t vh[NSTEP][NH2];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      Chunk<NWORDS> vcs = vc[s];
      if constexpr (APPEND && KV8) {
        if (masked && tok0 + RW * s >= last_start && rv)
          fix_step(vcs, TT * i + RW * s, s_pv, s_v, p.v_cache_w);
      }
      if constexpr (APPEND) {
        if (masked && tok0 + RW * s + row == newtok) vcs = vnew;
      }
      to_half_pairs<E, KV8>(vcs, vh[s]);
      if (masked) {
        const bool valid = tok0 + RW * s + row < L;
#pragma unroll
        for (int w = 0; w < NH2; ++w) vh[s][w] = valid ? vh[s][w] : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < NSTEP / 2; ++j) {
      uint32_t lo[NH2], hi[NH2];
#pragma unroll
      for (int w = 0; w < NH2; ++w) {
        lo[w] = __builtin_amdgcn_perm(vh[2 * j + 1][w], vh[2 * j][w], 0x05040100u);
        hi[w] = __builtin_amdgcn_perm(vh[2 * j + 1][w], vh[2 * j][w], 0x07060302u);
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float p0 = KV8 ? pw[2 * j][h] * vmul[2 * j] : pw[2 * j][h];
        const float p1 = KV8 ? pw[2 * j + 1][h] * vmul[2 * j + 1] : pw[2 * j + 1][h];
        const uint32_t pp = __builtin_bit_cast(uint32_t, half2_t{(_Float16)p0, (_Float16)p1});
#pragma unroll
        for (int w = 0; w < NH2; ++w) {
          acc[h][2 * w] = dot2(lo[w], pp, acc[h][2 * w]);
          acc[h][2 * w + 1] = dot2(hi[w], pp, acc[h][2 * w + 1]);
        }
      }
    }
  };

  // Tiles [0, n_full) are complete; tile n_full is the masked tail when the context ends
  // inside this wave's range. Two register buffers alternate so the next tile's loads are in
  // flight while the current one is consumed. The steady-state loop issues its loads
  // unconditionally: a conditional load would make the compiler's wait counts assume the
  // shorter queue and drain the prefetched tile before the current one is finished.
  const int avail = max(0, min(p0 + pn - wbase, share));
  int n_full = avail / TT;
  bool has_tail = (avail % TT) != 0;
  if constexpr (APPEND) {
    // the new token is the wave's last attended position: its tile takes the masked path,
    // which substitutes the new rows (a tile past the end masks nothing else)
    if (!has_tail && n_full > 0 && newtok >= wbase && newtok < wbase + avail) {
      --n_full;
      has_tail = true;
    }
  }
  const int n_tiles = n_full + (has_tail ? 1 : 0);
  if (n_tiles > 0) issue_tile(0, ka, va);
  int i = 0;
  if constexpr (APPEND && KV8) {
    // E4M3 append: every tile holding a position of the last block goes through the masked
    // path (blocks of up to 64 tokens, tiles of 16 or more tokens, aligned to the blocks)
    const int first_masked = max(0, (last_start - wbase) / TT);
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

  // ---- fused append: store the new rows at their slot ----------------------------------
  // Once per (sequence, KV head): the first head group's last partition, lanes 0 .. LPT-1 of
  // wave 0 (one row), and (E4M3) lane 0 the block's scales. Nothing in this launch reads the
  // slot's cached bytes for position L - 1, or those scales.
  if constexpr (APPEND) {
    if (appender && wave == 0 && lane < LPT) {
      const int64_t blk = new_slot / BS;
      const int off = (int)(new_slot - blk * BS);
      const size_t dst = ((size_t)blk * p.num_kv_heads + kvh) * TILE_BYTES +
                         (size_t)off * ROW_BYTES + (size_t)col * LANE_BYTES;
      store_chunk(p.k_cache_w + dst, knew);
      store_chunk(p.v_cache_w + dst, vnew);
      if (KV8 && lane == 0) {
        p.k_scale_w[(size_t)blk * p.num_kv_heads + kvh] = s_k;
        p.v_scale_w[(size_t)blk * p.num_kv_heads + kvh] = s_v;
      }
    }
  }

  // ---- the 16 / LPT tokens rows of a DPP row merge in registers (rotations by 8, then 4) ----
  if constexpr (LPT <= 8) merge_lane_states<0x128>(m, l, acc);  // row_ror:8
  if constexpr (LPT <= 4) merge_lane_states<0x124>(m, l, acc);  // row_ror:4

  // ---- merge the 4 DPP rows x kWaves waves of this workgroup through LDS ---------------
  // Lanes 0 .. LPT-1 of each DPP row now hold the whole row's state.
  constexpr int kDppRows = kWave / 16;
  auto s_acc = reinterpret_cast<float (*)[GT][D]>(lds);  // [kWaves * kDppRows][GT][D]
  auto s_ml = reinterpret_cast<float (*)[GT][2]>(lds + sizeof(float) * kWaves * kDppRows * GT * D);
  const int sub = wave * kDppRows + (lane >> 4);
  if ((lane & 15) < LPT) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[sub][h][col * E + e] = acc[h][e];
      if (col == 0) {
        s_ml[sub][h][0] = m[h];
        s_ml[sub][h][1] = l[h];
      }
    }
  }
  __syncthreads();

  // combine the 16 row states of this workgroup for element d of query head h
  auto local_merge = [&](int h, int d, float& mx, float& ls, float (&av)[1]) {
    float& a = av[0];
    mx = kNegInf;
#pragma unroll
    for (int k = 0; k < kWaves * kDppRows; ++k) mx = fmaxf(mx, s_ml[k][h][0]);
    const float ms = mx == kNegInf ? 0.f : mx;
    ls = 0.f;
    a = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves * kDppRows; ++k) {
      const float w = fexp2(s_ml[k][h][0] - ms);
      ls = fmaf(w, s_ml[k][h][1], ls);
      a = fmaf(w, s_acc[k][h][d], a);
    }
  };

  finish_partition<GT, D, kThreads, 1>(p, b, hg, part, nparts, sr.extra, h0, GT, local_merge);
}

template <int D, int BS, int GT, bool KV8, bool APPEND>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeParams p) {
  __shared__ __align__(16) uint8_t lds[decode_lds_bytes<D, GT>()];
  decode_body<D, BS, GT, KV8, APPEND>(p, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.y, lds);
}

template <int D, int BS, int GT, bool KV8, bool APPEND>
hipError_t launch_one(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads * p.head_groups, num_seqs, p.max_parts);
  decode_partition_kernel<D, BS, GT, KV8, APPEND><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, int BS, bool KV8, bool APPEND>
hipError_t dispatch_gt(const DecodeParams& p, int num_seqs, int gt, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_one<D, BS, 1, KV8, APPEND>(p, num_seqs, stream);
    case 2: return launch_one<D, BS, 2, KV8, APPEND>(p, num_seqs, stream);
    case 3: return launch_one<D, BS, 3, KV8, APPEND>(p, num_seqs, stream);
    case 4: return launch_one<D, BS, 4, KV8, APPEND>(p, num_seqs, stream);
    case 8:
      if constexpr (!KV8) return launch_one<D, BS, 8, KV8, APPEND>(p, num_seqs, stream);  // E4M3: at most 4
      break;
  }
  return hipErrorInvalidValue;
}

// ---- shared-prefix decode in one launch ---------------------------------------------------
// The first n_prefix workgroups are the prefix pass (the prefill body in its PREFIX form: each
// group's shared blocks once per KV head for the query rows of all members), the rest are the
// decode grid over the private tails (head group fastest, then grid row, then partition, as in
// decode_partition_kernel). The two kinds run side by side instead of one launch after the
// other; every partial goes to the workspace (deferred_merge = 2) and the merge kernel that
// follows on the stream combines them exactly.
template <int D, int BS, int GT, bool KV8, bool APPEND>
__global__ __launch_bounds__(kThreads, 2) void shared_prefix_decode_kernel(DecodeParams p,
                                                                        PrefillParams f,
                                                                        int n_prefix, int nseq) {
  constexpr size_t kPrefixLds = pf::prefill_lds_bytes<D, KV8, true>();
  constexpr size_t kDecodeLds = decode_lds_bytes<D, GT>();
  __shared__ __align__(16) uint8_t lds[kPrefixLds > kDecodeLds ? kPrefixLds : kDecodeLds];
  const int id = blockIdx.x;
  if (id < n_prefix) {
    pf::prefill_body<D, BS, KV8, true>(f, id, n_prefix, lds);
    return;
  }
  const int r = id - n_prefix;
  const int nx = p.num_kv_heads * p.head_groups;
  const int yz = r / nx;
  // cacheable K/V loads: members of a group read the same blocks (measured at 100 sequences
  // behind one 512-token prompt: 48.3 -> 42.4 us per step; after a fork, whose siblings share
  // their tails as well: 79.1 -> 67.6 us)
  decode_body<D, BS, GT, KV8, APPEND, false>(p, r - yz * nx, yz % nseq, yz / nseq, nseq, lds);
}

template <int D, int BS, int GT, bool KV8, bool APPEND>
hipError_t launch_sp(const DecodeParams& p, const PrefillParams& f, int n_prefix, int num_seqs,
                     hipStream_t stream) {
  const long long n = n_prefix + (long long)p.num_kv_heads * p.head_groups * num_seqs * p.max_parts;
  shared_prefix_decode_kernel<D, BS, GT, KV8, APPEND>
      <<<dim3((unsigned)n), kThreads, 0, stream>>>(p, f, n_prefix, num_seqs);
  return hipGetLastError();
}

template <int D, int BS, bool KV8, bool APPEND>
hipError_t sp_dispatch_gt(const DecodeParams& p, const PrefillParams& f, int n_prefix,
                          int num_seqs, int gt, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_sp<D, BS, 1, KV8, APPEND>(p, f, n_prefix, num_seqs, stream);
    case 2: return launch_sp<D, BS, 2, KV8, APPEND>(p, f, n_prefix, num_seqs, stream);
    case 3: return launch_sp<D, BS, 3, KV8, APPEND>(p, f, n_prefix, num_seqs, stream);
    case 4: return launch_sp<D, BS, 4, KV8, APPEND>(p, f, n_prefix, num_seqs, stream);
    case 8:
      if constexpr (!KV8) return launch_sp<D, BS, 8, KV8, APPEND>(p, f, n_prefix, num_seqs, stream);
      break;
  }
  return hipErrorInvalidValue;
}

template <int D, bool KV8, bool APPEND>
hipError_t sp_dispatch_bs(const DecodeParams& p, const PrefillParams& f, int n_prefix,
                          int num_seqs, int bs, int gt, hipStream_t stream) {
  switch (bs) {
    case 8: return sp_dispatch_gt<D, 8, KV8, APPEND>(p, f, n_prefix, num_seqs, gt, stream);
    case 16: return sp_dispatch_gt<D, 16, KV8, APPEND>(p, f, n_prefix, num_seqs, gt, stream);
    case 32: return sp_dispatch_gt<D, 32, KV8, APPEND>(p, f, n_prefix, num_seqs, gt, stream);
    case 64: return sp_dispatch_gt<D, 64, KV8, APPEND>(p, f, n_prefix, num_seqs, gt, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool KV8, bool APPEND>
hipError_t dispatch_bs(const DecodeParams& p, int num_seqs, int bs, int gt, hipStream_t stream) {
  switch (bs) {
    case 8: return dispatch_gt<D, 8, KV8, APPEND>(p, num_seqs, gt, stream);
    case 16: return dispatch_gt<D, 16, KV8, APPEND>(p, num_seqs, gt, stream);
    case 32: return dispatch_gt<D, 32, KV8, APPEND>(p, num_seqs, gt, stream);
    case 64: return dispatch_gt<D, 64, KV8, APPEND>(p, num_seqs, gt, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                         int head_tile, bool kv_fp8, hipStream_t stream) {
  if (head_dim == 128)
    return kv_fp8 ? dispatch_bs<128, true, false>(p, num_seqs, block_size, head_tile, stream)
                  : dispatch_bs<128, false, false>(p, num_seqs, block_size, head_tile, stream);
  if (head_dim == 64)
    return kv_fp8 ? dispatch_bs<64, true, false>(p, num_seqs, block_size, head_tile, stream)
                  : dispatch_bs<64, false, false>(p, num_seqs, block_size, head_tile, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_shared_prefix_decode(const DecodeParams& p, const PrefillParams& f,
                                       int n_prefix, int num_seqs, int head_dim, int block_size,
                                       int head_tile, bool kv_fp8, bool append,
                                       hipStream_t stream) {
  if (head_dim == 128) {
    if (kv_fp8) return sp_dispatch_bs<128, true, false>(p, f, n_prefix, num_seqs, block_size, head_tile, stream);
    return append ? sp_dispatch_bs<128, false, true>(p, f, n_prefix, num_seqs, block_size, head_tile, stream)
                  : sp_dispatch_bs<128, false, false>(p, f, n_prefix, num_seqs, block_size, head_tile, stream);
  }
  if (head_dim == 64) {
    if (kv_fp8) return sp_dispatch_bs<64, true, false>(p, f, n_prefix, num_seqs, block_size, head_tile, stream);
    return append ? sp_dispatch_bs<64, false, true>(p, f, n_prefix, num_seqs, block_size, head_tile, stream)
                  : sp_dispatch_bs<64, false, false>(p, f, n_prefix, num_seqs, block_size, head_tile, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_append(const DecodeParams& p, int num_seqs, int head_dim, int block_size,
                                int head_tile, bool kv_fp8, hipStream_t stream) {
  if (head_dim == 128)
    return kv_fp8 ? dispatch_bs<128, true, true>(p, num_seqs, block_size, head_tile, stream)
                  : dispatch_bs<128, false, true>(p, num_seqs, block_size, head_tile, stream);
  if (head_dim == 64)
    return kv_fp8 ? dispatch_bs<64, true, true>(p, num_seqs, block_size, head_tile, stream)
                  : dispatch_bs<64, false, true>(p, num_seqs, block_size, head_tile, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

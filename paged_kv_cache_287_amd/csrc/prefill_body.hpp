// Prefill workgroup body (see prefill_mfma.hip for the algorithm), shared by the prefill
// kernel and by the shared-prefix decode kernel, which runs prefix-pass workgroups in the same
// launch as the decode workgroups.
#pragma once

#include "decode_common.hpp"

namespace pa {
namespace pf {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int kWaveRows = 32;                        // query rows per wave (two 16-row tiles)
constexpr float kRescaleSlack = 8.f;                 // log2 units
constexpr int kTileTok = 64;                         // attended tokens per LDS tile
// Row padding (halves) of the K and V tiles in LDS ([token][d] rows). A 16-byte operand read
// takes 4 cycles per wave when its 64 addresses are spread over the banks and 8 when they pair
// up; rows of 256 + 32 bytes (D = 128) and 128 + 32 (D = 64) measured 4, rows padded by 16 bytes
// measured 8.
constexpr int kRowPad = 16;
static_assert(kPrefillRows == kWaves * kWaveRows, "rows per workgroup");

// Maximum of x over the four 16-lane rows of the wave (lanes lr, lr + 16, lr + 32, lr + 48),
// returned in every lane: two cross-row swaps, no LDS round trip. The IEEE maximum (NaN
// propagating; scores are never NaN for finite inputs) takes one v_maximum3 per swap, where
// fmaxf would first quiet both swapped operands.
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float y = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int NWORDS>
__device__ __forceinline__ h8 to_h8(const Chunk<NWORDS>& c) {
  uint32_t w[4];
  if constexpr (NWORDS == 4) {
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
}

// PREFIX selects the prefix pass of shared-prefix decode: the "sequences" are groups of decode
// sequences that share leading blocks, each member contributes its G query rows, every row sees
// all prefix tokens, and the prefix is cut into slices of prefix_split tokens, one workgroup
// each, whose unnormalised (max, sum, value sum) go to slots 0.. of the decode workspace.
// LDS of one prefill workgroup: the 64-token K and V tiles and the block ids of the attended
// range.
// An fp16 cache outside the prefix pass is staged by direct global -> LDS loads into two
// unpadded tile buffers (bank conflicts avoided by an XOR swizzle of the 16-byte chunks of a
// row); 8-bit caches, which need a conversion, and the prefix pass go through registers into
// one padded buffer.
template <bool KV8, bool PREFIX>
constexpr bool prefill_dma() {
  return !KV8 && !PREFIX;
}
template <int D, bool KV8, bool PREFIX>
constexpr size_t prefill_lds_bytes() {
  return (prefill_dma<KV8, PREFIX>() ? (size_t)(4 * kTileTok * D) * 2
                                     : (size_t)(2 * kTileTok * (D + kRowPad)) * 2) +
         (size_t)kPrefillMaxBlocks * 4;
}

// Physical 16-byte chunk slot of logical chunk c of tile row r in the unpadded buffers: c XOR
// swz(r). Rows hold D / 8 chunks (16 for D = 128, 8 for D = 64). swz moves the rows that share
// a bank range (every row at D = 128, every other row at D = 64) by distinct even slot counts,
// so the two chunks a transposed V read takes from a row stay adjacent. With it both operand
// reads ran without bank conflicts under the LDS counters (a K read 4 cycles per instruction,
// a transposed V read 2); the same XOR with a bit-0 term for rows 8..15 left the K reads 2-way
// conflicted.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 2 * (r & 7);
  else return 2 * ((r >> 1) & 3);
}

template <int D, int BS, bool KV8, bool PREFIX>
__device__ __forceinline__ void prefill_body(const PrefillParams& p, int wid_in, int nwg,
                                             uint8_t* lds) {
  constexpr int NT = kWaveRows / 16;
  constexpr int KK = D / 32;              // 32-dim steps of S^T = K Q^T
  constexpr int MT = D / 16;              // 16-dim tiles of O^T
  constexpr int ESZ = KV8 ? 1 : 2;
  constexpr int ROW_BYTES = D * ESZ;
  constexpr int TILE_BYTES = BS * ROW_BYTES;  // one block of one KV head
  constexpr int NWORDS = 2 * ESZ;         // 32-bit words per 8-element chunk
  constexpr int DCH = D / 8;              // 8-element chunks per token row
  constexpr int TPT = kTileTok * DCH / kThreads;  // consecutive tokens staged per thread (4 or 2)
  constexpr int KRS = D + kRowPad;        // LDS row stride of K (halves)
  constexpr int VRS = D + kRowPad;        // LDS row stride of V (halves)
  static_assert(TPT == 4 || TPT == 2, "staging shape");

  constexpr bool DMA = prefill_dma<KV8, PREFIX>();
  // LDS (prefill_lds_bytes): [K tile][V tile]([K tile][V tile] with DMA)[block ids]
  _Float16* k_lds = reinterpret_cast<_Float16*>(lds);
  _Float16* v_lds = k_lds + kTileTok * (DMA ? D : KRS);
  int32_t* ids = reinterpret_cast<int32_t*>(k_lds + kTileTok * (DMA ? 4 * D : KRS + VRS));
  constexpr int kBuf = kTileTok * 2 * D;  // halves between the two DMA buffers (K and V pairs)

  // ---- which (sequence, KV head, row tile): consecutive ids on one XCD share a KV range ------
  int wid = wid_in;
  const int per_xcd = nwg / kNumXcds;
  if (wid < per_xcd * kNumXcds) wid = (wid % kNumXcds) * per_xcd + wid / kNumXcds;
  const int qt = p.q_tiles - 1 - wid % p.q_tiles;  // later rows attend more: dispatched first
  const int kvh = (wid / p.q_tiles) % p.num_kv_heads;
  const int unit = wid / (p.q_tiles * p.num_kv_heads);
  // prefix pass: a unit is (group, slice of prefix_split tokens of its prefix)
  const int b = PREFIX ? unit / p.prefix_slices : unit;
  const int slice = PREFIX ? unit - b * p.prefix_slices : 0;

  const int T = p.num_tokens;
  const int qs = min(max(p.query_start[b], 0), T);
  const int qe = min(max(p.query_start[b + 1], qs), T);
  const int n = min(qe - qs, p.max_query_len);
  const int G = p.group;
  const int nrows = n * G;
  const int row0 = qt * kPrefillRows;
  if (row0 >= nrows) return;  // uniform over the workgroup
  int base, kv_begin = 0, kv_end;
  if constexpr (PREFIX) {
    // the decode pass derives the same clamp and slice count from the same inputs
    const int total = min(p.group_prefix_blocks[b], p.max_prefix_blocks) * BS;
    kv_begin = slice * p.prefix_split;
    if (kv_begin >= total) return;  // no prefix, or fewer slices than the grid allows for
    kv_end = min(total, kv_begin + p.prefix_split);
    base = total - 1;     // every row sees the whole prefix
  } else {
    const int L = min(max(p.context_lens[b], 0), p.max_context_len);
    base = L - n;         // position of the chunk's first token
    kv_end = max(0, min(L, base + (min(row0 + kPrefillRows, nrows) - 1) / G + 1));
  }
  // table row: the sequence's own, or (prefix pass) the group's first member's
  const int32_t* table = p.block_tables + (size_t)(PREFIX ? qs : b) * p.max_blocks_per_seq;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lq = lane >> 4;

  // ---- block ids of the attended range ------------------------------------------------------
  // (kv_begin is a multiple of the 64-token tile, hence of the block size)
  const int blk0 = kv_begin / BS;
  const int nblk = (kv_end + BS - 1) / BS - blk0;
  for (int i = tid; i < nblk; i += kThreads) {
    ids[i] = min(max(table[blk0 + i], 0), p.num_blocks - 1);
  }

  // ---- this wave's query rows as the B operand of S^T = K Q^T -------------------------------
  // A negative softmax scale is applied as |scale| with the query negated (exact in fp16), so
  // the per-score multiplier is positive and the row max can be taken before scaling.
  const float qscale = fabsf(p.scale_log2);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  const int wrow0 = row0 + wave * kWaveRows;
  h8 qb[NT][KK];
  int pos[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = wrow0 + 16 * nt + lr;
    const bool ok = r < nrows;
    const int j = ok ? r / G : 0;
    const int h = kvh * G + (ok ? r - j * G : 0);
    pos[nt] = ok ? (PREFIX ? base : base + j) : -1;
    const _Float16* qrow = p.q + ((size_t)(qs + j) * p.num_q_heads + h) * D + 8 * lq;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w = ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * kk) : u32x4{0, 0, 0, 0};
      w ^= qsign;
      qb[nt][kk] = __builtin_bit_cast(h8, w);
    }
  }
  // positions of the wave's first and last valid rows (rows are in token order)
  const int wpos_lo = PREFIX ? base : base + wrow0 / G;
  const int wpos_hi =
      wrow0 < nrows ? (PREFIX ? base : base + (min(wrow0 + kWaveRows, nrows) - 1) / G) : -1;

  // m: running maximum (the reference of l and o); nms and mlim: -m (0 while m is -inf) and
  // m + kRescaleSlack, kept beside it so a tile without a rescale does not recompute them
  float m[NT], l[NT], nms[NT], mlim[NT];
  f4 o[NT][MT], osum[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = kNegInf;
    nms[nt] = 0.f;
    mlim[nt] = kNegInf;
    l[nt] = 0.f;
    osum[nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nt][mt] = f4{0.f, 0.f, 0.f, 0.f};
  }
  // A operand whose row 0 is all ones (lanes lr == 0 hold row 0's eight slots)
  const _Float16 one = lr == 0 ? (_Float16)1.f : (_Float16)0.f;
  const h8 ones = h8{one, one, one, one, one, one, one, one};

  // ---- staging: thread -> (TPT consecutive tokens, one 8-element chunk of d) ------------------
  const int sch = tid % DCH;
  const int st0 = (tid / DCH) * TPT;
  const uint8_t* kbase = p.k_cache + (size_t)kvh * TILE_BYTES + sch * 8 * ESZ;
  const uint8_t* vbase = p.v_cache + (size_t)kvh * TILE_BYTES + sch * 8 * ESZ;
  const size_t blk_stride = (size_t)p.num_kv_heads * TILE_BYTES;
  Chunk<NWORDS> kr[TPT], vr[TPT];

  // A thread's TPT tokens start at a multiple of 4, so they share one block (block sizes are
  // multiples of 8): one id lookup per tile. Tokens past kv_end re-read the last token before
  // it (in bounds; masked later).
  auto issue = [&](int tile) {
    const int t0 = tile * kTileTok + st0;
    if (tile * kTileTok + kTileTok <= kv_end) {
      // whole tile inside the range (uniform): one address, constant row offsets
      const size_t off = (size_t)ids[t0 / BS - blk0] * blk_stride + (size_t)(t0 % BS) * ROW_BYTES;
      const uint8_t* kp = kbase + off;
      const uint8_t* vp = vbase + off;
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        kr[u] = load_chunk<NWORDS>(kp + u * ROW_BYTES);
        vr[u] = load_chunk<NWORDS>(vp + u * ROW_BYTES);
      }
      return;
    }
    const int tc = min(t0, kv_end - 1);
    const int last = max(0, kv_end - 1 - t0);
    const size_t off = (size_t)ids[tc / BS - blk0] * blk_stride + (size_t)(tc % BS) * ROW_BYTES;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const size_t o = off + (size_t)min(u, last) * ROW_BYTES;
      kr[u] = load_chunk<NWORDS>(kbase + o);
      vr[u] = load_chunk<NWORDS>(vbase + o);
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      *reinterpret_cast<h8*>(k_lds + (st0 + u) * KRS + 8 * sch) = to_h8(kr[u]);
      *reinterpret_cast<h8*>(v_lds + (st0 + u) * VRS + 8 * sch) = to_h8(vr[u]);
    }
  };

  // masked: the tile reaches some row's causal limit (a uniform branch around the selects)
  // per-lane swizzle terms of the operand reads (rows 16 s + lr; rows 4 lq + lr / 4 (+16))
  const int xk = DMA ? swz<D>(lr) ^ lq : 0;
  const int xv = DMA ? swz<D>(4 * lq + (lr >> 2)) ^ ((lr & 3) >> 1) : 0;
  auto compute = [&](int tile, bool masked, int buf) {
    const int tok0 = tile * kTileTok;
    const _Float16* kt = k_lds + buf;
    const _Float16* vtl = v_lds + buf;
    float kmul[4], vmul[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kmul[s] = qscale;
      vmul[s] = 1.f;
      if constexpr (KV8) {
        // a lane's four tokens 16s + 4lq .. +3 share one block (block sizes are multiples of 4)
        const int id = ids[min(tok0 + 16 * s + 4 * lq, kv_end - 1) / BS - blk0];
        kmul[s] *= p.k_scale[(size_t)id * p.num_kv_heads + kvh];
        vmul[s] = p.v_scale[(size_t)id * p.num_kv_heads + kvh];
      }
    }
    // S^T for the four 16-token sub-tiles and both row tiles
    // (32-dim step outermost: the 4 x NT products of one step are independent, so the matrix
    // cores never wait on a previous product's result)
    f4 sacc[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[nt][s] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      h8 kA[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (DMA)
          kA[s] = *reinterpret_cast<const h8*>(kt + (16 * s + lr) * D + 8 * ((4 * kk) ^ xk));
        else
          kA[s] = *reinterpret_cast<const h8*>(kt + (16 * s + lr) * KRS + 32 * kk + 8 * lq);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          sacc[nt][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[s], qb[nt][kk], sacc[nt][s], 0, 0, 0);
    }
    // online softmax per row (lane lr's row; its 16 tokens of the tile are spread over lq)
    h8 pB[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // raw scores; the multiplier goes into the exponent's fma (and, with one multiplier for
      // the whole tile, after the max)
      float sv[4][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sv[s][ii] = sacc[nt][s][ii];
      if (masked) {
        const int lim = pos[nt] - tok0 - 4 * lq;  // token 16 s + ii of the lane is past it
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            if (16 * s + ii > lim) sv[s][ii] = kNegInf;
      }
      float tm = kNegInf;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) tm = fmaxf(tm, KV8 ? sv[s][ii] * kmul[s] : sv[s][ii]);
      if constexpr (!KV8) tm *= qscale;
      tm = row4_max(tm);
      // the running max is the reference of l and o; it moves (with a rescale) only when a
      // score passes it by more than kRescaleSlack (wave-uniform decision), so most tiles skip
      // the rescale; probabilities stay below 2^kRescaleSlack
      if (__builtin_amdgcn_ballot_w64(tm > mlim[nt]) != 0) {
        const float mn = fmaxf(m[nt], tm);
        const float alpha = fexp2(m[nt] - (mn == kNegInf ? 0.f : mn));
        l[nt] *= alpha;
        if constexpr (!KV8) osum[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
        m[nt] = mn;
        nms[nt] = mn == kNegInf ? 0.f : -mn;
        mlim[nt] = mn + kRescaleSlack;
      }
      float pw[4][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) pw[s][ii] = fexp2(fmaf(sv[s][ii], kmul[s], nms[nt]));
      if constexpr (KV8) {
        // the probabilities going to the matrix cores carry the V scale, so the row sums are
        // taken here; without it they come out of the P.V product (osum)
        float ps = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) ps += pw[s][ii];
        l[nt] += ps;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int s0 = 2 * ks, s1 = 2 * ks + 1;
        pB[nt][ks] = h8{(_Float16)(pw[s0][0] * vmul[s0]), (_Float16)(pw[s0][1] * vmul[s0]),
                        (_Float16)(pw[s0][2] * vmul[s0]), (_Float16)(pw[s0][3] * vmul[s0]),
                        (_Float16)(pw[s1][0] * vmul[s1]), (_Float16)(pw[s1][1] * vmul[s1]),
                        (_Float16)(pw[s1][2] * vmul[s1]), (_Float16)(pw[s1][3] * vmul[s1])};
      }
    }
    // O^T += V^T P^T, 32 tokens per product; for an fp16 cache one more product with an
    // all-ones row in place of V^T accumulates the row sums of P (osum, element 0 of lanes
    // lq == 0), on the matrix cores instead of 32 adds per tile
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // The A operand is V^T: lane (lr, lq) holds dim 16 mt + lr of the tokens its eight
        // contraction slots stand for (those of its P^T slots: 32 ks + 4 lq + 0..3, then the
        // same + 16). ds_read_b64_tr_b16 reads it from the row-major V tile: within each
        // 16-lane group, lane j passes 4 halves of a row and lane i receives, as its element e,
        // half i % 4 of lane (4 e + i / 4)'s row; lane lr therefore passes the row of token
        // 32 ks + 4 lq + lr / 4 at dims 16 mt + 4 (lr % 4) .. + 3, and one read covers four
        // tokens.
        typedef short s4 __attribute__((ext_vector_type(4)));
        constexpr int RS = DMA ? D : VRS;
        const _Float16* src =
            DMA ? vtl + (32 * ks + 4 * lq + (lr >> 2)) * D + 8 * ((2 * mt) ^ xv) + 4 * (lr & 1)
                : vtl + (32 * ks + 4 * lq + (lr >> 2)) * VRS + 16 * mt + 4 * (lr & 3);
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(src));
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(src + 16 * RS));
        const h8 vA = __builtin_bit_cast(h8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vA, pB[nt][ks], o[nt][mt], 0, 0, 0);
      }
      if constexpr (!KV8) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          osum[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pB[nt][ks], osum[nt], 0, 0, 0);
      }
    }
  };

  __syncthreads();  // ids visible
  const int tile_lo = kv_begin / kTileTok;
  const int tile_hi = (kv_end + kTileTok - 1) / kTileTok;
  if constexpr (DMA) {
    // Direct loads: one instruction moves 1 KB (RPI rows) into LDS, lane l's 16 bytes to byte
    // 16 l, so lane l loads logical chunk (l % CPR) ^ swz(row) of its row. Wave w fills rows
    // 16 w .. 16 w + 15 of each tile with NI instructions for K and NI for V.
    constexpr int CPR = D / 8;
    constexpr int RPI = 1024 / ROW_BYTES;
    constexpr int NI = 16 / RPI;
    int loff[NI];  // byte offset of a lane's chunk in its block's tile (rows within one block)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int t = 16 * wave + RPI * j + lane / CPR;
      loff[j] = (t % BS) * ROW_BYTES + 16 * ((lane % CPR) ^ swz<D>(t));
    }
    const uint8_t* kh = p.k_cache + (size_t)kvh * TILE_BYTES;
    const uint8_t* vh = p.v_cache + (size_t)kvh * TILE_BYTES;
    auto dma = [&](int tile, int buf) {
      typedef __attribute__((address_space(3))) void* lds_ptr;
      if (tile * kTileTok + kTileTok <= kv_end) {
        // whole tile in range: the RPI rows of one instruction sit in one block (BS >= 8), and
        // the wave's 16 rows in one block unless BS is 8 (then in two)
        constexpr int NB = BS >= 16 ? 1 : 2;
        int bid[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k)
          bid[k] = __builtin_amdgcn_readfirstlane(
              ids[(tile * kTileTok + 16 * wave + 8 * k) / BS - blk0]);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int row = 16 * wave + RPI * j;
          const size_t bo = (size_t)bid[NB == 1 ? 0 : (RPI * j) / 8] * blk_stride;
          __builtin_amdgcn_global_load_lds(kh + bo + loff[j], (lds_ptr)(k_lds + buf + row * D),
                                           16, 0, 0);
          __builtin_amdgcn_global_load_lds(vh + bo + loff[j], (lds_ptr)(v_lds + buf + row * D),
                                           16, 0, 0);
        }
      } else {
        // last tile: rows past kv_end load the last attended token again (finite; masked)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int row = 16 * wave + RPI * j;
          const int t = row + lane / CPR;
          const int tok = min(tile * kTileTok + t, kv_end - 1);
          const size_t o = (size_t)ids[tok / BS - blk0] * blk_stride +
                           (size_t)(tok % BS) * ROW_BYTES + 16 * ((lane % CPR) ^ swz<D>(t));
          __builtin_amdgcn_global_load_lds(kh + o, (lds_ptr)(k_lds + buf + row * D), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vh + o, (lds_ptr)(v_lds + buf + row * D), 16, 0, 0);
        }
      }
    };
    // tile i sits in buffer (i - tile_lo) % 2; the loop takes two tiles per trip so that each
    // buffer's LDS offsets are constants folded into the read instructions
    auto step = [&](int i, int buf) {
      // this wave's loads of tile i have landed; after the barrier every wave's have, and every
      // wave is done with tile i - 1, whose buffer the next loads overwrite
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (i + 1 < tile_hi) dma(i + 1, kBuf - buf);
      const int tok0 = i * kTileTok;
      if (tok0 > wpos_hi) return;  // every token of the tile is in this wave's causal future
      compute(i, tok0 + kTileTok - 1 > wpos_lo, buf);
    };
    if (tile_lo < tile_hi) dma(tile_lo, 0);
    for (int i = tile_lo; i < tile_hi; i += 2) {
      step(i, 0);
      if (i + 1 < tile_hi) step(i + 1, kBuf);
    }
  } else {
    if (tile_lo < tile_hi) issue(tile_lo);
    for (int i = tile_lo; i < tile_hi; ++i) {
      __syncthreads();  // every wave is done reading the previous tile
      stage();
      __syncthreads();
      if (i + 1 < tile_hi) issue(i + 1);
      const int tok0 = i * kTileTok;
      if (tok0 > wpos_hi) continue;  // every token of the tile is in this wave's causal future
      compute(i, tok0 + kTileTok - 1 > wpos_lo, 0);
    }
  }

  // ---- normalise and write this wave's rows ------------------------------------------------
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt;
    if constexpr (KV8) {
      lt = l[nt];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
    } else {
      lt = __shfl(osum[nt][0], lr);  // row lr's sum sits in lane lr (lq == 0), element 0
    }
    const int r = wrow0 + 16 * nt + lr;
    if (r >= nrows) continue;
    const int j = r / G;
    const int h = kvh * G + (r - j * G);
    if constexpr (PREFIX) {
      // slot `slice` of (member qs + j, head h), for the decode pass that follows on the same
      // stream to merge; the kernel boundary makes these plain stores visible to it
      const size_t slot = ((size_t)(qs + j) * p.num_q_heads + h) * p.part_slots + slice;
      float* acc = p.ws_acc + slot * D + 4 * lq;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f4*>(acc + 16 * mt) = o[nt][mt];
      if (lq == 0) *reinterpret_cast<f2*>(p.ws_ml + slot * 2) = f2{m[nt], lt};
      continue;
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    _Float16* orow = p.out + ((size_t)(qs + j) * p.num_q_heads + h) * D + 4 * lq;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<h4*>(orow + 16 * mt) =
          h4{(_Float16)(o[nt][mt][0] * inv), (_Float16)(o[nt][mt][1] * inv),
             (_Float16)(o[nt][mt][2] * inv), (_Float16)(o[nt][mt][3] * inv)};
  }
}

}  // namespace pf
}  // namespace pa

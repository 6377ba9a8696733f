// Device helpers shared by the decode kernels (VALU and MFMA): loads, E4M3 decoding, and the end
// of a partition (direct write, or publish + merge by the last workgroup to arrive).
#pragma once

#include "pa_internal.hpp"

namespace pa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A product the compiler may not fuse with a later add. A score s * k feeds both the running
// maximum and the exponent 2^(s * k - m); fused into the exponent in unmasked tiles but not in
// masked ones (where a select sits between them), the same token would round differently
// depending on the tile's path. Kept separate, the result depends only on the values, and the
// exponent of the maximum's own token is exactly 0.
__device__ __forceinline__ float mul_nc(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Two OCP E4M3 codes (bytes 0-1, or 2-3 with hi) -> two fp16, exactly: every E4M3 value,
// subnormals included, is representable in fp16, and the NaN code decodes to NaN. gfx950's
// conversion uses the OCP encoding (checked against the format's definition for all 256 codes).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Partials of one partition are read by whichever workgroup finishes a sequence last, possibly on
// another XCD (each XCD has its own L2). System-scope relaxed accesses compile to write-through
// stores and cache-bypassing loads (sc0 sc1), which keeps that exchange coherent without
// flushing any cache.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Maximum over groups of LPT consecutive lanes (4, 8 or 16) of a DPP row; every lane of a group
// receives it.
template <int LPT>
__device__ __forceinline__ float lane_group_max(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "lane group");
  x = fmaxf(x, dpp_mov<0xB1>(x));                           // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));                           // quad_perm [2,3,0,1]
  if constexpr (LPT >= 8) x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
  if constexpr (LPT >= 16) x = fmaxf(x, dpp_mov<0x140>(x)); // row_mirror
  return x;
}

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

template <int NWORDS>
struct Chunk {
  uint32_t w[NWORDS];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// NT = non-temporal: KV bytes are read once per call, so they are streamed past the caches
// (measured on MI355X: ~7.0 TB/s for a non-temporal streaming read vs ~6.3 TB/s without).
template <int NWORDS, bool NT = false>
__device__ __forceinline__ Chunk<NWORDS> load_chunk(const uint8_t* ptr) {
  Chunk<NWORDS> c;
  if constexpr (NWORDS == 4) {
    const u32x4* p = reinterpret_cast<const u32x4*>(ptr);
    const u32x4 v = NT ? __builtin_nontemporal_load(p) : *p;
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else if constexpr (NWORDS == 2) {
    const u32x2* p = reinterpret_cast<const u32x2*>(ptr);
    const u32x2 v = NT ? __builtin_nontemporal_load(p) : *p;
    c.w[0] = v.x; c.w[1] = v.y;
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(ptr);
    c.w[0] = NT ? __builtin_nontemporal_load(p) : *p;
  }
  return c;
}

template <int NWORDS>
__device__ __forceinline__ void store_chunk(uint8_t* ptr, const Chunk<NWORDS>& c) {
  if constexpr (NWORDS == 4) {
    *reinterpret_cast<u32x4*>(ptr) = u32x4{c.w[0], c.w[1], c.w[2], c.w[3]};
  } else if constexpr (NWORDS == 2) {
    *reinterpret_cast<u32x2*>(ptr) = u32x2{c.w[0], c.w[1]};
  } else {
    *reinterpret_cast<uint32_t*>(ptr) = c.w[0];
  }
}

// Context range [start, L) of sequence b covered by this call's partitions, and the number of
// partial slots that an earlier pass already filled for it. Plain decode covers the whole
// context. With shared-prefix groups, a member of a group with a non-empty prefix starts after
// the prefix blocks, whose partials the prefix pass stored in slots 0 .. extra - 1 (one per
// slice of prefix_split tokens).
struct SeqRange {
  int L, start, extra;
};
template <int BS>
__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int b) {
  SeqRange r{p.context_lens[b], 0, 0};
  if (p.group_start != nullptr) {
    // last group whose first sequence is <= b
    int lo = 0, hi = p.num_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.group_start[mid] <= b) lo = mid;
      else hi = mid - 1;
    }
    const bool member = p.group_start[lo] <= b && b < p.group_start[lo + 1];
    // the same clamp as the prefix pass (at most max_prefix_blocks, itself within the table
    // and the prefix pass's on-chip id list); shared blocks beyond it are decoded per sequence
    const int pb = member ? min(p.group_prefix_blocks[lo], p.max_prefix_blocks) : 0;
    if (pb > 0) {
      r.start = min(pb * BS, max(r.L, 0));
      r.extra = (pb * BS + p.prefix_split - 1) / p.prefix_split;
    }
  }
  return r;
}

// Write-through 16-byte store of a partial (system scope: it leaves the writer's L2 for memory,
// where a workgroup on another XCD reads it with cache-bypassing loads). A vector store.
__device__ __forceinline__ void publish4(float* p, const float (&v)[4]) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v x = f4v{v[0], v[1], v[2], v[3]};
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" : : "v"(p), "v"(x) : "memory");
}
// Two adjacent floats of a partial with one cache-bypassing 8-byte load.
__device__ __forceinline__ void fetch2(const float* p, float& x, float& y) {
  const unsigned long long w = __hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_SYSTEM);
  x = __builtin_bit_cast(float, (uint32_t)w);
  y = __builtin_bit_cast(float, (uint32_t)(w >> 32));
}

// End of one (sequence, head group, partition) workgroup. merge(h, d0, mx, ls, a) returns the
// workgroup's combined running max, running sum and weighted value sums for elements
// d0 .. d0 + UE - 1 of its query row h (the first `rows` of R rows, head dim D). A thread takes
// UE consecutive elements at a time and neighbouring threads take neighbouring elements, so
// every store and load below is contiguous across a wave (UE = 4: 16 bytes per lane). With one
// partition and no earlier partial the normalised output is written directly; otherwise the
// partial is published (after the `extra` slots an earlier pass filled) and the workgroup that
// arrives last merges all slots exactly and resets the arrival counter to zero (or, with
// deferred_merge, a kernel of its own merges them).
template <int R, int D, int NTHREADS, int UE, typename Merge>
__device__ __forceinline__ void finish_partition(const DecodeParams& p, int b, int hg, int part,
                                                 int nparts, int extra, int h0, int rows,
                                                 Merge&& merge) {
  static_assert(UE == 1 || UE == 4, "one element or 16 bytes of partial per item");
  typedef float f4v __attribute__((ext_vector_type(4)));
  typedef _Float16 h4v __attribute__((ext_vector_type(4)));
  constexpr int IPR = D / UE;  // items per row
  const int tid = threadIdx.x;
  const int items = rows * IPR;
  // normalised output of one item: one 2-byte or one 8-byte store
  auto write_out = [&](int h, int d0, const float (&a)[UE], float ls) {
    _Float16* o = p.out + ((size_t)b * p.num_q_heads + h0 + h) * D + d0;
    if constexpr (UE == 4) {
      h4v v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = (_Float16)(ls > 0.f ? a[u] / ls : 0.f);
      *reinterpret_cast<h4v*>(o) = v;
    } else {
      o[0] = (_Float16)(ls > 0.f ? a[0] / ls : 0.f);
    }
  };
  if (nparts == 1 && extra == 0) {
    // the whole sequence fits one partition: normalise and write the output directly
    for (int it = tid; it < items; it += NTHREADS) {
      const int h = it / IPR, d0 = (it - h * IPR) * UE;
      float mx, ls, a[UE];
      merge(h, d0, mx, ls, a);
      write_out(h, d0, a, ls);
    }
    return;
  }
  if (nparts == 1 && p.deferred_merge != 2) {
    // this launch's only partition of the sequence plus the `extra` partials an earlier launch
    // (the shared-prefix pass) stored: merge them here and write the output, with no publish of
    // this partition and no arrival count (the earlier kernel's stores are visible to plain
    // loads in this one)
    for (int it = tid; it < items; it += NTHREADS) {
      const int h = it / IPR, d0 = (it - h * IPR) * UE;
      float mx, ls, a[UE];
      merge(h, d0, mx, ls, a);
      const size_t row0 = ((size_t)b * p.num_q_heads + h0 + h) * p.part_slots;
      float mv[kMaxPrefixSlices], lv[kMaxPrefixSlices], av[kMaxPrefixSlices][UE];
#pragma unroll
      for (int j = 0; j < kMaxPrefixSlices; ++j) {
        const bool in = j < extra;
        const size_t slot = row0 + (in ? j : 0);
        mv[j] = in ? p.ws_ml[slot * 2] : kNegInf;
        lv[j] = in ? p.ws_ml[slot * 2 + 1] : 0.f;
        if constexpr (UE == 4) {
          const f4v x = *reinterpret_cast<const f4v*>(p.ws_acc + slot * D + d0);
#pragma unroll
          for (int u = 0; u < 4; ++u) av[j][u] = in ? x[u] : 0.f;  // unused slots: anything
        } else {
          av[j][0] = in ? p.ws_acc[slot * D + d0] : 0.f;
        }
      }
      float mc = mx;
#pragma unroll
      for (int j = 0; j < kMaxPrefixSlices; ++j) mc = fmaxf(mc, mv[j]);
      const float ms = mc == kNegInf ? 0.f : mc;
      const float w0 = fexp2(mx - ms);
      ls *= w0;
#pragma unroll
      for (int u = 0; u < UE; ++u) a[u] *= w0;
#pragma unroll
      for (int j = 0; j < kMaxPrefixSlices; ++j) {
        const float w = fexp2(mv[j] - ms);
        ls = fmaf(w, lv[j], ls);
#pragma unroll
        for (int u = 0; u < UE; ++u) a[u] = fmaf(w, av[j][u], a[u]);
      }
      write_out(h, d0, a, ls);
    }
    return;
  }

  // ---- several partitions: publish this one's (max, sum, value sum) ----------------------
  for (int it = tid; it < items; it += NTHREADS) {
    const int h = it / IPR, d0 = (it - h * IPR) * UE;
    float mx, ls, a[UE];
    merge(h, d0, mx, ls, a);
    const size_t slot = ((size_t)b * p.num_q_heads + h0 + h) * p.part_slots + extra + part;
    float* dst = p.ws_acc + slot * D + d0;
    if (p.deferred_merge) {
      // the merge kernel that follows on the stream reads them: plain stores, no counter
      if constexpr (UE == 4) *reinterpret_cast<f4v*>(dst) = f4v{a[0], a[1], a[2], a[3]};
      else dst[0] = a[0];
    } else {
      if constexpr (UE == 4) publish4(dst, a);
      else publish(dst, a[0]);
    }
    if (d0 == 0) {
      if (p.deferred_merge) {
        p.ws_ml[slot * 2] = mx;
        p.ws_ml[slot * 2 + 1] = ls;
      } else {
        publish(p.ws_ml + slot * 2, mx);
        publish(p.ws_ml + slot * 2 + 1, ls);
      }
    }
  }
  if (p.deferred_merge) return;
  // Count arrivals once the partial is stored. The workgroup that arrives last merges every
  // partition of this (sequence, head group) and resets the counter to zero, so no second
  // kernel is needed and the counters are zero again for the next call. The partials go
  // through write-through stores and come back through cache-bypassing loads (see publish /
  // fetch); every wave waits for its stores to complete (s_waitcnt 0) before the barrier, so
  // the counter only moves once the whole partial is in memory. No L2 write-back or
  // invalidation is needed (those cost far more than the merge itself).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    int32_t* ctr = p.counters + (size_t)b * p.num_kv_heads * p.head_groups + hg;
    const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nparts - 1;
    if (s_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;

  // exact merge: out = sum_p 2^(m_p - M) a_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
  // A thread takes IPT items of 4 consecutive dims (neighbouring threads, neighbouring dims).
  // The partitions are taken KC at a time with the loads of all IPT items in flight together
  // (each round trip is a full memory latency: the loads bypass the caches), and merged into a
  // running (max, sum, value) exactly as the tiles were.
  constexpr int IT_ROW = D / 4;
  constexpr int IPT = (R * IT_ROW + NTHREADS - 1) / NTHREADS;
  constexpr int KC = IPT >= 4 ? 4 : 8;
  const int nslots = nparts + extra;
  int hs[IPT], ds[IPT];
  bool act[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int it = tid + k * NTHREADS;
    act[k] = it < rows * IT_ROW;
    hs[k] = act[k] ? it / IT_ROW : 0;
    ds[k] = act[k] ? (it - hs[k] * IT_ROW) * 4 : 0;
  }
  float mx[IPT], ls[IPT], a[IPT][4];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    mx[k] = kNegInf;
    ls[k] = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) a[k][u] = 0.f;
  }
  for (int i0 = 0; i0 < nslots; i0 += KC) {
    float mv[IPT][KC], lv[IPT][KC], av[IPT][KC][4];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const size_t row0 = ((size_t)b * p.num_q_heads + h0 + hs[k]) * p.part_slots;
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const bool in = i0 + j < nslots;
        const size_t slot = row0 + (in ? i0 + j : i0);
        fetch2(p.ws_ml + slot * 2, mv[k][j], lv[k][j]);
        fetch2(p.ws_acc + slot * D + ds[k], av[k][j][0], av[k][j][1]);
        fetch2(p.ws_acc + slot * D + ds[k] + 2, av[k][j][2], av[k][j][3]);
        if (!in) mv[k][j] = kNegInf;
      }
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      float mc = mx[k];
#pragma unroll
      for (int j = 0; j < KC; ++j) mc = fmaxf(mc, mv[k][j]);
      const float r = fexp2(mx[k] - mc);  // mx = -inf only before the first chunk: r = 0
      ls[k] *= r;
#pragma unroll
      for (int u = 0; u < 4; ++u) a[k][u] *= r;
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const float w = fexp2(mv[k][j] - mc);
        ls[k] = fmaf(w, lv[k][j], ls[k]);
#pragma unroll
        for (int u = 0; u < 4; ++u) a[k][u] = fmaf(w, av[k][j][u], a[k][u]);
      }
      mx[k] = mc;
    }
  }
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    if (!act[k]) continue;
    h4v v;
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (_Float16)(a[k][u] / ls[k]);
    *reinterpret_cast<h4v*>(p.out + ((size_t)b * p.num_q_heads + h0 + hs[k]) * D + ds[k]) = v;
  }
}

}  // namespace pa

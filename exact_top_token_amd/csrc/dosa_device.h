// Device-side building blocks for gfx950: MFMA operand fragments, ordered
// 64-bit candidate keys and the wavefront radix select.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dosa_internal.h"

namespace dosa {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

typedef unsigned long long u64;

// ---------------------------------------------------------------------------
// Candidate keys.  A candidate (score, key position) is packed into one u64
// whose unsigned order is the selection order: score descending, then
// position ascending.  High word: the float's bits mapped to an unsigned
// total order; low word: ~position.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f2ord(float f) {
  // negative: all bits flipped; otherwise the sign bit set (three VALU ops)
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ u64 make_key(float s, int pos) {
  return ((u64)f2ord(s) << 32) | (u64)(uint32_t)(~(uint32_t)pos);
}
__device__ __forceinline__ int key_pos(u64 e) { return (int)(~(uint32_t)e); }
__device__ __forceinline__ float key_score(u64 e) { return ord2f((uint32_t)(e >> 32)); }

// Two fp8 E4M3FN codes (bytes 2*HI, 2*HI+1 of w) -> two bf16 in one word,
// low half first.  gfx950's converter with scale 1: every finite E4M3 value
// (subnormals m*2^-9 included) is a bf16 value, so the result is exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  const v2bf_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// MFMA operand fragments.  For a 16x16xK MFMA, lane l supplies row (A) or
// column (B) l%16; lane group g = l/16 supplies its share of the reduction
// dimension.  Both operands use the same assignment: lane group g owns the
// contiguous elements [g*d/4, (g+1)*d/4) of every row, split into STEPS
// instructions, so each MFMA output is a full-length dot product.
// ---------------------------------------------------------------------------
template <int C, int D>
struct Ops;

template <int D>
struct Ops<C_F32, D> {
  static constexpr int STEPS = D / 4;
  static constexpr int QB = 4, KB = 4;
  typedef float frag;
  __device__ __forceinline__ static void load_q(const void* row, int g, frag* f) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + g * (D / 4));
#pragma unroll
    for (int v = 0; v < D / 16; ++v) {
      float4 t = p[v];
      f[4 * v] = t.x; f[4 * v + 1] = t.y; f[4 * v + 2] = t.z; f[4 * v + 3] = t.w;
    }
  }
  __device__ __forceinline__ static void load_k(const void* row, int g, frag* f) { load_q(row, g, f); }
  __device__ __forceinline__ static void zero(frag* f) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) f[s] = 0.f;
  }
  __device__ __forceinline__ static v4f mma(frag a, frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct Ops<C_BF16, D> {
  static constexpr int STEPS = D / 32;
  static constexpr int QB = 2, KB = 2;
  typedef v8bf frag;
  __device__ __forceinline__ static void load_q(const void* row, int g, frag* f) {
    const v4i* p = reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(row) + g * (D / 4));
#pragma unroll
    for (int s = 0; s < STEPS; ++s) f[s] = __builtin_bit_cast(v8bf, p[s]);
  }
  __device__ __forceinline__ static void load_k(const void* row, int g, frag* f) { load_q(row, g, f); }
  __device__ __forceinline__ static void zero(frag* f) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) f[s] = __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
  }
  __device__ __forceinline__ static v4f mma(frag a, frag b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct Ops<C_FP8, D> {
  static constexpr int STEPS = 1;
  static constexpr int QB = 1, KB = 1;
  typedef v8i frag;
  __device__ __forceinline__ static void load_q(const void* row, int g, frag* f) {
    const uint8_t* b = static_cast<const uint8_t*>(row);
    if constexpr (D == 128) {
      const v4i* p = reinterpret_cast<const v4i*>(b + 32 * g);
      v4i lo = p[0], hi = p[1];
      f[0] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v4i* p = reinterpret_cast<const v4i*>(b + 16 * g);
      v4i lo = p[0];
      f[0] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ static void load_k(const void* row, int g, frag* f) { load_q(row, g, f); }
  __device__ __forceinline__ static void zero(frag* f) { f[0] = v8i{0, 0, 0, 0, 0, 0, 0, 0}; }
  // this lane's d/4 key bytes as loaded (zero-padded to 32), and their fragments
  typedef v8i raw;
  __device__ __forceinline__ static void load_raw(const void* row, int g, raw& r) { load_q(row, g, &r); }
  __device__ __forceinline__ static void from_raw(const raw& r, frag* f) { f[0] = r; }
  __device__ __forceinline__ static v4f mma(frag a, frag b, v4f c) {
    // operand formats 0/0 = fp8 E4M3 for A and B; scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// bf16 queries against fp8 keys: keys are widened to bf16 (exact) in registers.
template <int D>
struct Ops<C_BF16Q_FP8K, D> {
  static constexpr int STEPS = D / 32;
  static constexpr int QB = 2, KB = 1;
  typedef v8bf frag;
  __device__ __forceinline__ static void load_q(const void* row, int g, frag* f) {
    Ops<C_BF16, D>::load_q(row, g, f);
  }
  __device__ __forceinline__ static void load_k(const void* row, int g, frag* f) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(row) + g * (D / 4));
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      uint32_t w0 = p[2 * s], w1 = p[2 * s + 1];
      v4i v;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w = h ? w1 : w0;
        v[2 * h] = (int)fp8x2_to_bf16x2<false>(w);
        v[2 * h + 1] = (int)fp8x2_to_bf16x2<true>(w);
      }
      f[s] = __builtin_bit_cast(v8bf, v);
    }
  }
  __device__ __forceinline__ static void zero(frag* f) { Ops<C_BF16, D>::zero(f); }
  __device__ __forceinline__ static v4f mma(frag a, frag b, v4f c) { return Ops<C_BF16, D>::mma(a, b, c); }
  // this lane's d/4 key bytes as loaded (zero-padded to 32), and their fragments
  typedef v8i raw;
  __device__ __forceinline__ static void load_raw(const void* row, int g, raw& r) {
    Ops<C_FP8, D>::load_raw(row, g, r);
  }
  __device__ __forceinline__ static void from_raw(const raw& r, frag* f) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      v4i v;
      v[0] = (int)fp8x2_to_bf16x2<false>((uint32_t)r[2 * s]);
      v[1] = (int)fp8x2_to_bf16x2<true>((uint32_t)r[2 * s]);
      v[2] = (int)fp8x2_to_bf16x2<false>((uint32_t)r[2 * s + 1]);
      v[3] = (int)fp8x2_to_bf16x2<true>((uint32_t)r[2 * s + 1]);
      f[s] = __builtin_bit_cast(v8bf, v);
    }
  }
};

// Key operands that can be prefetched as raw bytes one step ahead (fp8 keys:
// 32 bytes per lane and 16-key block).
template <int C>
struct KeyRaw { static constexpr bool value = (C == C_FP8 || C == C_BF16Q_FP8K); };

template <int C>
struct HasQScale { static constexpr bool value = (C == C_FP8); };
template <int C>
struct HasKScale { static constexpr bool value = (C == C_FP8 || C == C_BF16Q_FP8K); };

// Queries per wavefront for a (combo, H, d): the largest of 4/2/1 whose
// register-resident query rows fit 128 VGPRs and whose head slots (16/QW)
// divide H.  MFMA row r = (query r/(16/QW), head slot r%(16/QW)).
__host__ __device__ constexpr int queries_per_wave(int C, int H, int D) {
  int qb = (C == C_F32) ? 4 : (C == C_FP8 ? 1 : 2);
  int per = H * D * qb;
  if (4 * per <= 32768 && H % 4 == 0) return 4;
  if (2 * per <= 32768 && H % 8 == 0) return 2;
  return 1;
}

// ---------------------------------------------------------------------------
// Key addressing (contiguous or paged storage)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t key_row(const Inputs& in, int key_base, int seq, int key) {
  if (in.page_table == nullptr) return (int64_t)key_base + key;
  if (in.page_shift >= 0) {   // power-of-two pages: shift and mask instead of an integer division
    const int pg = in.page_table[(int64_t)seq * in.max_pages + (key >> in.page_shift)];
    return ((int64_t)pg << in.page_shift) + (key & (in.page_size - 1));
  }
  const int pg = in.page_table[(int64_t)seq * in.max_pages + key / in.page_size];
  return (int64_t)pg * in.page_size + key % in.page_size;
}

// ---------------------------------------------------------------------------
// Wavefront helpers (one 64-lane wavefront per workgroup)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The lane id computed afresh where it is used.  Values derived from it are
// then recomputed in place instead of being hoisted out of the scoring loops
// and held in registers (two VALU instructions instead of a spill).
__device__ __forceinline__ int lane_fresh() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// Lane mask of a per-lane condition.  Takes the condition as a bool, so a
// comparison result goes straight into the mask (HIP's __ballot takes an int
// and materialises it in a vector register first).
__device__ __forceinline__ unsigned long long ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

// Wait until every memory operation this wavefront has issued is complete.
// Placed after the loads that set up a prefetching loop, it keeps the
// compiler from merging their pending state into the loop, where its wait
// for them would also wait for each iteration's own prefetch.
__device__ __forceinline__ void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Wait for this wavefront's vector memory operations only (vmcnt(0); the LDS
// and export counters at their maxima).  Unconditional, so the compiler knows
// afterwards that no load is pending on any path.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Memory fence plus wavefront barrier: this wavefront's LDS and global
// writes are visible to its own later reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t o = __shfl_down(v, off, 64);
    if (lane + off < 64) v += o;
  }
  return v;
}

// Squared norm (of the stored values, before any per-key scale) of the key
// in this lane's column, from the key block's MFMA fragments: B^T B of the 16
// keys has their squared norms on its diagonal, and column c's entry is
// element c%4 of lane 16*(c/4) + c.  Products of stored values are exact in
// fp32 and every term is nonnegative, so the fp32 sum is within d*2^-24 of
// the exact value.  All 64 lanes must take part (one lane exchange).
template <class O>
__device__ __forceinline__ float frag_norm2(const typename O::frag* B) {
  v4f gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < O::STEPS; ++s) gm = O::mma(B[s], B[s], gm);
  const int l = lane_id(), c = l & 15, e = c & 3;
  float dv = (e == 0) ? gm[0] : (e == 1) ? gm[1] : (e == 2) ? gm[2] : gm[3];
  dv = ((l >> 4) == (c >> 2)) ? dv : 0.f;
  return __shfl(dv, 16 * (c >> 2) + c, 64);
}

// Upper bound on ||k|| (stored values) from frag_norm2: sqrt, then rounded up
// by 2^-16 relative, which covers the fp32 sum of d <= 128 squares and the sqrt.
__device__ __forceinline__ float norm_up(float n2) { return sqrtf(n2) * 1.0000153f; }

// Wavefront-rows of 64 candidates loaded together by the streaming loops.
constexpr int kBatch = 8;

// Segmented view of a query's candidate regions.
// The regions r0.. of one query: entries and counts of region r0 + r.
struct Segs {
  const u64* base;         // the query's row in region r0
  const uint32_t* counts;  // the query's count in region r0
  int64_t rstride;         // entries from one region's row to the next
  int64_t cstride;         // counts from one region to the next
  int nseg;
  uint32_t cap;            // entries a region holds: a count is never read as more
  const uint32_t* off;     // LDS [nseg + 1]: prefix sums of the (clamped) counts, or NULL
  __device__ __forceinline__ uint32_t n(int r) const { return min(counts[(int64_t)r * cstride], cap); }
  __device__ __forceinline__ const u64* ptr(int r) const { return base + (int64_t)r * rstride; }
};

// Queries with more segments than this are read as one flattened index range
// (many short regions: one segment's loads at a time would serialise their
// latencies); with fewer, segment by segment (cheaper per entry).
constexpr int kFlatSegments = 8;

// The prefix sums of a query's segment counts into LDS off[0..nseg] (thread 0;
// the caller synchronises before use).  With them, a pass over the query's
// entries runs over one flattened index range with the loads of all segments
// in flight together, instead of one segment after the other.
__device__ __forceinline__ void segment_offsets(const Segs& sg, uint32_t* off) {
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int r = 0; r < sg.nseg; ++r) {
      off[r] = a;
      a += sg.n(r);
    }
    off[sg.nseg] = a;
  }
}

// The same prefix sums by all NT threads of the workgroup: the counts are
// loaded in parallel (one thread's loop over them waits out a memory latency
// per segment, which dominates queries of many short segments), then
// wavefront 0 scans them.  Synchronises the workgroup before returning.
template <int NT>
__device__ __forceinline__ void segment_offsets_wg(const Segs& sg, uint32_t* off) {
  const int tid = (int)threadIdx.x;
  for (int r = tid; r < sg.nseg; r += NT) off[r + 1] = sg.n(r);
  __syncthreads();
  if (tid < 64) {
    uint32_t carry = 0;
    for (int c = 0; c < sg.nseg; c += 64) {
      const int r = c + tid;
      uint32_t v = r < sg.nseg ? off[r + 1] : 0u;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = (uint32_t)__shfl_up((int)v, o, 64);
        if (tid >= o) v += u;
      }
      if (r < sg.nseg) off[r + 1] = carry + v;
      carry += (uint32_t)__shfl((int)v, 63, 64);
    }
    if (tid == 0) off[0] = 0u;
  }
  __syncthreads();
}

// K-th largest of the (distinct) entries of the segments, K >= 1 and
// K <= total, by a workgroup of NT threads.  Radix select on 11/11/10-bit
// digits from the top; stops as soon as the digit bin holding the K-th entry
// is taken whole.  Returns T with exactly K entries >= T (the same value in
// every wavefront: each reads the shared histogram and decides alike).
// hist: 2048 u32 of LDS.
template <int NT>
__device__ __noinline__ u64 select_kth_nt(const Segs sg, int K, uint32_t* hist) {
  const int lane = lane_id();
  const int tid = (int)threadIdx.x;
  u64 prefix = 0;
  uint32_t rem = (uint32_t)K;
  __syncthreads();
#pragma unroll 1
  for (int p = 0; p < 6; ++p) {
    const int sh = (p == 0) ? 53 : (p == 1) ? 42 : (p == 2) ? 32 : (p == 3) ? 21 : (p == 4) ? 10 : 0;
    const int wd = (p == 2 || p == 5) ? 10 : 11;
    const int nb = 1 << wd;
    const int hs = sh + wd;
    for (int b = tid; b < nb; b += NT) hist[b] = 0;
    __syncthreads();
    const u64 want = (p == 0) ? 0 : (prefix >> hs);
    if (sg.off != nullptr && sg.nseg > kFlatSegments) {
      // one flattened index range over all segments (a thread's indices only
      // grow, so its segment cursor only moves forward)
      const uint32_t total = sg.off[sg.nseg];
      int r = 0;
      for (uint32_t b = 0; b < total; b += NT * kBatch) {
        u64 e[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {     // all loads of the batch in flight together
          const uint32_t i = b + (uint32_t)NT * u + tid;
          e[u] = 0ull;
          if (i < total) {
            while (sg.off[r + 1] <= i) ++r;
            e[u] = sg.ptr(r)[i - sg.off[r]];
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = b + (uint32_t)NT * u + tid;
          if (i < total && (p == 0 || (e[u] >> hs) == want))
            atomicAdd(&hist[(uint32_t)(e[u] >> sh) & (uint32_t)(nb - 1)], 1u);
        }
      }
    } else {
      for (int r = 0; r < sg.nseg; ++r) {
        const u64* ptr = sg.ptr(r);
        const uint32_t n = sg.n(r);
        for (uint32_t b = 0; b < n; b += NT * kBatch) {
          u64 e[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {     // all loads of the batch in flight together
            const uint32_t i = b + (uint32_t)NT * u + tid;
            e[u] = (i < n) ? ptr[i] : 0ull;
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const uint32_t i = b + (uint32_t)NT * u + tid;
            if (i < n && (p == 0 || (e[u] >> hs) == want))
              atomicAdd(&hist[(uint32_t)(e[u] >> sh) & (uint32_t)(nb - 1)], 1u);
          }
        }
      }
    }
    __syncthreads();
    const int per = nb >> 6;
    uint32_t s = 0;
    for (int t = 0; t < per; ++t) s += hist[lane * per + t];
    const uint32_t suf = wave_suffix_sum(s);
    const bool cross = (suf >= rem) && (suf - s < rem);
    const u64 cm = __ballot(cross);
    const int L = cm ? (__ffsll((long long)cm) - 1) : 0;
    uint32_t acc = __shfl(suf - s, L, 64);
    int b = L * per;
    uint32_t cnt_b = 0;
    for (int t = per - 1; t >= 0; --t) {
      const uint32_t h = hist[L * per + t];
      if (acc + h >= rem) { b = L * per + t; cnt_b = h; break; }
      acc += h;
    }
    rem -= acc;
    prefix |= ((u64)(uint32_t)b) << sh;
    __syncthreads();
    if (cnt_b == rem) break;
  }
  return prefix;
}

__device__ __forceinline__ u64 select_kth(const Segs sg, int K, uint32_t* hist) { return select_kth_nt<64>(sg, K, hist); }

// Copy the entries >= T of src[0..n) to dst[out..] in order (dst may equal
// src, with out <= 0 then).  Returns the new end.  Entries are read kBatch
// wavefront-rows at a time before any is written: in place, every write
// lands below the first unread entry, so the batch cannot clobber its input.
__device__ __forceinline__ uint32_t compact_ge(const u64* src, uint32_t n, u64 T, u64* dst, uint32_t out) {
  const int lane = lane_id();
  for (uint32_t base = 0; base < n; base += 64 * kBatch) {
    u64 e[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = base + 64u * u + lane;
      e[u] = (i < n) ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = base + 64u * u + lane;
      const bool keep = (i < n) && (e[u] >= T);
      const u64 m = __ballot(keep);
      const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
      if (keep) dst[out + before] = e[u];
      out += __popcll(m);
    }
  }
  return out;
}

// compact_ge, also lowering mn (wavefront-uniform on return) to the smallest
// entry kept.  When exactly K entries are >= T, that is the K-th largest.
__device__ __forceinline__ uint32_t compact_ge_min(const u64* src, uint32_t n, u64 T, u64* dst, uint32_t out,
                                                   u64& mn) {
  const int lane = lane_id();
  u64 m_lane = mn;
  for (uint32_t base = 0; base < n; base += 64 * kBatch) {
    u64 e[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = base + 64u * u + lane;
      e[u] = (i < n) ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = base + 64u * u + lane;
      const bool keep = (i < n) && (e[u] >= T);
      const u64 m = __ballot(keep);
      const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
      if (keep) {
        dst[out + before] = e[u];
        m_lane = e[u] < m_lane ? e[u] : m_lane;
      }
      out += __popcll(m);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const u64 o = __shfl_xor(m_lane, off, 64);
    m_lane = o < m_lane ? o : m_lane;
  }
  mn = m_lane;
  return out;
}

}  // namespace dosa

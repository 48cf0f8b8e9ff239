// Final merge of the candidate regions: the exact Top-K per query, and the
// dispatch of the scoring launchers by operand combination.
#include "dosa_device.h"

namespace dosa {

// ---------------------------------------------------------------------------
// final merge: the exact Top-K of each query over regions [r0, r1)
// ---------------------------------------------------------------------------
constexpr int kMaxMergeRegions = 256;   // regions whose offsets the merge keeps in LDS

// Entries >= T among src[0..n), counted by one wavefront.
__device__ __forceinline__ uint32_t count_ge(const u64* src, uint32_t n, u64 T) {
  const int lane = lane_id();
  uint32_t c = 0;
  for (uint32_t b0 = 0; b0 < n; b0 += 64 * kBatch) {
    u64 e[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = b0 + 64u * u + lane;
      e[u] = (i < n) ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = b0 + 64u * u + lane;
      c += (uint32_t)__popcll(__ballot((i < n) && (e[u] >= T)));
    }
  }
  return c;
}

// One wavefront writes the entries >= T of src[0..n), in order, to rows
// out.. of oi / os (positions and scores), none at or past K.  Returns the
// next free row.
__device__ __forceinline__ uint32_t emit_ge(const u64* src, uint32_t n, u64 T, int32_t* oi, float* os,
                                            uint32_t out, int K) {
  const int lane = lane_id();
  for (uint32_t b0 = 0; b0 < n; b0 += 64 * kBatch) {
    u64 e[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = b0 + 64u * u + lane;
      e[u] = (i < n) ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t i = b0 + 64u * u + lane;
      const bool keep = (i < n) && (e[u] >= T);
      const u64 m = __ballot(keep);
      const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
      if (keep && out + before < (uint32_t)K) {
        oi[out + before] = key_pos(e[u]);
        if (os) os[out + before] = key_score(e[u]);
      }
      out += __popcll(m);
    }
  }
  return out;
}

// NT threads per query: the radix passes use them all; the compaction and
// the output walk stay on wavefront 0 (its order is the regions' order, so
// rows are the same run to run).  NT = 256 serves launches with few queries,
// whose time is one query's latency.
template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(const SelectLaunch p) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t segoff[kMaxMergeRegions + 1];
  constexpr int NW = NT / 64;
  __shared__ uint32_t woff[NW];
  if (skip_launch(p.mode, p.run_if)) return;
  const int q = p.q_first + blockIdx.x;
  const int lane = lane_id();
  const int K = p.topk;
  const u64* base = p.cb.row(q, p.r0);
  const uint32_t* cnt = p.cb.count(q, p.r0);
  const int nseg = ((p.mode != nullptr && *p.mode == MODE_UNPRUNED) ? p.r1_unpruned : p.r1) - p.r0;
  Segs sg{base, cnt, p.cb.rows * p.cb.cap, p.cb.rows, nseg, (uint32_t)p.cb.cap, nullptr};
  if (nseg <= kMaxMergeRegions) {
    segment_offsets_wg<NT>(sg, segoff);
    sg.off = segoff;
  }
  uint32_t total = 0;
  if (sg.off != nullptr) total = sg.off[nseg];
  else
    for (int r = 0; r < nseg; ++r) total += sg.n(r);
  u64 T = 0;
  if (total >= (uint32_t)K) T = select_kth_nt<NT>(sg, K, hist);
  if (p.out_idx == nullptr) {
    // threshold mode: keep only the K entries >= T in the merged regions, so
    // a later merge reads K of them instead of all.  T is the lower edge of
    // the radix bin that holds the K-th entry; the smallest kept entry is the
    // K-th largest itself, and its score is the threshold tau.
    if (threadIdx.x >= 64) return;
    u64 mn = ~0ull;
    if (total >= (uint32_t)K) {
      for (int r = 0; r < nseg; ++r) {
        u64* ptr = p.cb.row(q, p.r0 + r);
        const uint32_t nk = compact_ge_min(ptr, sg.n(r), T, ptr, 0, mn);
        wave_sync();   // every lane has read the count before lane 0 rewrites it
        if (lane == 0) *p.cb.count(q, p.r0 + r) = nk;
      }
    }
    const float tau = (total >= (uint32_t)K) ? key_score(mn) : -INFINITY;
    if (lane == 0) {
      if (p.tau_out != nullptr) p.tau_out[q] = tau;
      if (p.tau_copy != nullptr) p.tau_copy[q] = tau;
      if (p.coef_tau != nullptr) p.coef_tau[(int64_t)q * kCoefStride + 5] = tau;
    }
    return;
  }
  // exactly min(K, total) entries are >= T; write them in flattened order
  // (region by region), which is the same run to run
  int32_t* oi = p.out_idx + (int64_t)q * K;
  float* os = p.out_score ? p.out_score + (int64_t)q * K : nullptr;
  uint32_t out = 0;
  if (NW > 1 && sg.off != nullptr) {
    // Each wavefront takes one contiguous share of the flattened entries: it
    // counts its entries >= T, the counts become output offsets in order, and
    // each share is written at its offset.
    const int w = (int)(threadIdx.x >> 6);
    const uint32_t lo = (uint32_t)((uint64_t)total * w / NW), hi = (uint32_t)((uint64_t)total * (w + 1) / NW);
    int r0 = 0;
    while (r0 < nseg && sg.off[r0 + 1] <= lo) ++r0;
    uint32_t c = 0;
    for (int r = r0; r < nseg && sg.off[r] < hi; ++r) {
      const uint32_t s0 = max(lo, sg.off[r]) - sg.off[r], s1 = min(hi, sg.off[r + 1]) - sg.off[r];
      c += count_ge(sg.ptr(r) + s0, s1 - s0, T);
    }
    if (lane == 0) woff[w] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t acc = 0;
      for (int i = 0; i < NW; ++i) {
        const uint32_t v = woff[i];
        woff[i] = acc;
        acc += v;
      }
    }
    __syncthreads();
    uint32_t o = woff[w];
    for (int r = r0; r < nseg && sg.off[r] < hi; ++r) {
      const uint32_t s0 = max(lo, sg.off[r]) - sg.off[r], s1 = min(hi, sg.off[r + 1]) - sg.off[r];
      o = emit_ge(sg.ptr(r) + s0, s1 - s0, T, oi, os, o, K);
    }
    out = min(total, (uint32_t)K);
    for (uint32_t i = out + threadIdx.x; i < (uint32_t)K; i += NT) {
      oi[i] = -1;
      if (os) os[i] = -INFINITY;
    }
    return;
  }
  if (threadIdx.x >= 64) return;
  for (int r = 0; r < nseg; ++r) out = emit_ge(sg.ptr(r), sg.n(r), T, oi, os, out, K);
  out = min(out, (uint32_t)K);
  for (uint32_t i = out + lane; i < (uint32_t)K; i += 64) {
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
}

// Same merge, rows ordered by (score desc, position asc): the kept keys are
// gathered into LDS and bitonic-sorted (K <= 4096 -> 32 KiB).
__global__ __launch_bounds__(64) void select_sorted_kernel(const SelectLaunch p) {
  __shared__ uint32_t hist[2048];
  __shared__ u64 keys[4096];
  if (skip_launch(p.mode, p.run_if)) return;
  const int q = p.q_first + blockIdx.x;
  const int lane = lane_id();
  const int K = p.topk;
  const u64* base = p.cb.row(q, p.r0);
  const uint32_t* cnt = p.cb.count(q, p.r0);
  const int nseg = ((p.mode != nullptr && *p.mode == MODE_UNPRUNED) ? p.r1_unpruned : p.r1) - p.r0;
  const Segs sg{base, cnt, p.cb.rows * p.cb.cap, p.cb.rows, nseg, (uint32_t)p.cb.cap, nullptr};
  uint32_t total = 0;
  for (int r = 0; r < nseg; ++r) total += sg.n(r);
  u64 T = 0;
  if (total >= (uint32_t)K) T = select_kth(sg, K, hist);
  if (p.tau_out != nullptr && lane == 0) p.tau_out[q] = (total >= (uint32_t)K) ? key_score(T) : -INFINITY;
  int N = 1;
  while (N < K) N <<= 1;
  for (int i = lane; i < N; i += 64) keys[i] = 0ull;
  __syncthreads();
  uint32_t out = 0;
  for (int r = 0; r < nseg; ++r) {
    const u64* src = sg.ptr(r);
    const uint32_t n = sg.n(r);
    for (uint32_t b0 = 0; b0 < n; b0 += 64 * kBatch) {
      u64 e[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = b0 + 64u * u + lane;
        e[u] = (i < n) ? src[i] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = b0 + 64u * u + lane;
        const bool keep = (i < n) && (e[u] >= T);
        const u64 m = __ballot(keep);
        const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
        if (keep && out + before < (uint32_t)K) keys[out + before] = e[u];
        out += __popcll(m);
      }
    }
  }
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = lane; i < (N >> 1); i += 64) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const u64 a = keys[lo], b = keys[hi];
        if (desc ? (a < b) : (a > b)) { keys[lo] = b; keys[hi] = a; }
      }
      __syncthreads();
    }
  }
  int32_t* oi = p.out_idx + (int64_t)q * K;
  float* os = p.out_score ? p.out_score + (int64_t)q * K : nullptr;
  out = min(out, (uint32_t)K);
  for (int i = lane; i < K; i += 64) {
    const bool real = (uint32_t)i < out;
    const u64 e = keys[i];
    oi[i] = real ? key_pos(e) : -1;
    if (os) os[i] = real ? key_score(e) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_score_f32(int H, int d, const ScoreLaunch& p, hipStream_t s);
hipError_t launch_score_bf16(int H, int d, const ScoreLaunch& p, hipStream_t s);
hipError_t launch_score_fp8(int H, int d, const ScoreLaunch& p, hipStream_t s);
hipError_t launch_score_bf16fp8(int H, int d, const ScoreLaunch& p, hipStream_t s);

hipError_t launch_score(int combo, int H, int d, const ScoreLaunch& p, hipStream_t s) {
  switch (combo) {
    case C_F32: return launch_score_f32(H, d, p, s);
    case C_BF16: return launch_score_bf16(H, d, p, s);
    case C_FP8: return launch_score_fp8(H, d, p, s);
    case C_BF16Q_FP8K: return launch_score_bf16fp8(H, d, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectLaunch& p, hipStream_t s) {
  if (p.total_q == 0) return hipSuccess;
  if (p.sorted && p.out_idx != nullptr)
    hipLaunchKernelGGL(select_sorted_kernel, dim3(p.total_q), dim3(64), 0, s, p);
  else if (p.total_q <= 256)
    hipLaunchKernelGGL((select_kernel<1024>), dim3(p.total_q), dim3(1024), 0, s, p);
  else if (p.total_q <= 2048)
    hipLaunchKernelGGL((select_kernel<256>), dim3(p.total_q), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((select_kernel<64>), dim3(p.total_q), dim3(64), 0, s, p);
  return hipGetLastError();
}

int tile_waves() { return kTileWaves; }

bool combo_supported(int combo, int H, int d) {
  if (combo < 0 || combo > 3) return false;
  if (!(d == 64 || d == 128)) return false;
  if (H < 8 || H > 64 || H % 8 != 0) return false;   // kernels built for 8/16/32/64 head slots
  return true;
}

}  // namespace dosa

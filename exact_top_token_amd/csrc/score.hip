// Exact all-head scoring on MFMA with a streaming per-query candidate buffer.
//
// One wavefront scores one query group (QW consecutive queries of a sequence)
// against a list of keys.  MFMA rows are (query, head slot) pairs, columns are
// 16 keys, the reduction runs over the head dimension d:
//     x[(t,h), s] = q[t,h,:] . k[s,:]            (fp32 accumulation)
// and each lane folds its 4 output rows -- 4 heads of one query -- into
//     S(t,s) = sum_h w[t,h] * max(0, x)           (then x q_scale * k_scale)
// so after all head groups every lane holds a finished score with no
// cross-lane reduction (QW = 4; QW = 2/1 need one/two lane exchanges).
//
// Scores at or above the query's running threshold theta are appended to the
// query's candidate region as packed (score, position) keys.  When a region
// nears its capacity the wavefront runs an exact radix select over it,
// keeps the current K best and raises theta to the K-th score (prior art named
// by the DoSA pages, Related Work: radix selection and bounded-buffer
// streaming; DoSA Method section: fuse full scoring with threshold filtering
// and pack scores for selection).
#include "dosa_device.h"

namespace dosa {

template <int C, int H, int D>
__global__ __launch_bounds__(64) void score_kernel(const ScoreLaunch p) {
  using O = Ops<C, D>;
  constexpr int QW = queries_per_wave(C, H, D);
  constexpr int S = 16 / QW;   // head slots per query in one MFMA
  constexpr int HG = H / S;    // head groups
  constexpr int STEPS = O::STEPS;
  __shared__ uint32_t hist[2048];

  const int lane = lane_id();
  const WorkItem it = p.items[blockIdx.x];
  const GroupInfo gr = p.groups[it.group];
  const int col = lane & 15;   // key column (B operand and outputs)
  const int g = lane >> 4;     // lane group

  // Query rows of this group, kept in registers for the whole key sweep.
  typename O::frag A[HG][STEPS];
  {
    const int ra = lane & 15;
    const int qa = ra / S, hs = ra % S;
    const bool ok = qa < gr.nq;
    const uint8_t* qb = static_cast<const uint8_t*>(p.in.q);
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      const int head = S * j + hs;
      if (ok)
        O::load_q(qb + ((int64_t)(gr.q_row0 + qa) * H + head) * D * O::QB, g, A[j]);
      else
        O::zero(A[j]);
    }
  }
  // Weights of this lane's output rows: rows 4g..4g+3 belong to query qi.
  const int qi = (4 * g) / S;
  const bool qok = qi < gr.nq;
  const int qrow = gr.q_row0 + qi;
  float wv[HG][4];
#pragma unroll
  for (int j = 0; j < HG; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = S * j + ((4 * g + i) % S);
      wv[j][i] = qok ? p.in.w[(int64_t)qrow * H + head] : 0.f;
    }
  const float qs = (HasQScale<C>::value && qok) ? p.in.q_scale[qrow] : 1.f;
  const int pos = gr.pos0 + qi;
  float theta = (p.theta_init != nullptr && qok) ? p.theta_init[qrow] : -INFINITY;
  uint32_t count = 0;
  const int owner_lane0 = 16 * (qi * (4 / QW));
  const bool owner = (lane >> 4) == (owner_lane0 >> 4);
  const int R = p.cb.R, cap = p.cb.cap;
  u64* const cand_base = p.cb.cand;
  u64* const buf = qok ? cand_base + ((int64_t)qrow * R + it.region) * cap : nullptr;
  const uint32_t hi_water = (uint32_t)(cap - 16);
  uint32_t n_written = 0, n_reselect = 0, n_scored = 0;

  const uint8_t* kbytes = static_cast<const uint8_t*>(p.in.k);

  auto block = [&](int key, bool kvalid) {
    typename O::frag B[STEPS];
    float ks = 1.f;
    if (kvalid) {
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      O::load_k(kbytes + row * D * O::KB, g, B);
      if constexpr (HasKScale<C>::value) ks = p.in.k_scale[row];
    } else {
      O::zero(B);
    }
    float o = 0.f;
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s) c = O::mma(A[j][s], B[s], c);
#pragma unroll
      for (int i = 0; i < 4; ++i) o += wv[j][i] * fmaxf(c[i], 0.f);
    }
    if constexpr (QW <= 2) o += __shfl_xor(o, 16, 64);
    if constexpr (QW == 1) o += __shfl_xor(o, 32, 64);
    const float score = o * qs * ks;
    const bool valid = owner && qok && kvalid && key <= pos;
    const bool take = valid && score >= theta;
    const u64 m = __ballot(take);
    n_scored += __popcll(__ballot(valid));
    const uint32_t slice = (uint32_t)(m >> owner_lane0) & 0xFFFFu;
    const uint32_t before = __popc(slice & ((1u << col) - 1u));
    if (take) buf[count + before] = make_key(score, key);
    count += __popc(slice);
    n_written += __popcll(m);
    if (__any(count > hi_water)) {
#pragma unroll 1
      for (int qq = 0; qq < QW; ++qq) {
        const int src = 16 * (qq * (4 / QW));
        const uint32_t cq = __shfl(count, src, 64);
        if (cq > hi_water) {
          u64* bq = cand_base + ((int64_t)(gr.q_row0 + qq) * R + it.region) * cap;
          uint32_t one = cq;
          Segs s1{bq, &one, cap, 1};
          const u64 T = select_kth(s1, p.topk, hist);
          compact_ge(bq, cq, T, bq, 0);
          __syncthreads();
          if (qi == qq) {
            count = (uint32_t)p.topk;
            theta = key_score(T);
          }
          ++n_reselect;
        }
      }
    }
  };

  if (!it.gather) {
#pragma unroll 1
    for (int r = 0; r < 2; ++r) {
      const int lo = r ? it.b0 : it.a0, hi = r ? it.b1 : it.a1;
#pragma unroll 1
      for (int kb = hi - 16; kb > lo - 16; kb -= 16) {
        const int key = kb + col;
        block(key, key >= lo && key < hi);
      }
    }
  } else {
    const int32_t* lst = p.lists + gr.list_off;
    const int len = p.list_len[it.group];
    const int e0 = (int)(((int64_t)len * it.a0 / it.a1) & ~15LL);
    const int e1 = (it.a0 == it.a1 - 1) ? len : (int)(((int64_t)len * (it.a0 + 1) / it.a1) & ~15LL);
#pragma unroll 1
    for (int e = e0; e < e1; e += 16) {
      const int idx = e + col;
      const bool kv = idx < e1;
      const int key = kv ? lst[idx] : 0;
      block(key, kv);
    }
  }

  if (qok && lane == owner_lane0) p.cb.counts[(int64_t)qrow * R + it.region] = count;
  if (p.stats != nullptr && lane == 0) {
    atomicAdd(&p.stats[p.scored_slot], (u64)n_scored);
    atomicAdd(&p.stats[5], (u64)n_written);
    atomicAdd(&p.stats[6], (u64)n_reselect);
  }
}

// Final merge: the exact Top-K of each query over regions [r0, r1).
__global__ __launch_bounds__(64) void select_kernel(const SelectLaunch p) {
  __shared__ uint32_t hist[2048];
  const int q = blockIdx.x;
  const int lane = lane_id();
  const int R = p.cb.R, cap = p.cb.cap, K = p.topk;
  const u64* base = p.cb.cand + ((int64_t)q * R + p.r0) * cap;
  const uint32_t* cnt = p.cb.counts + (int64_t)q * R + p.r0;
  const int nseg = p.r1 - p.r0;
  uint32_t total = 0;
  for (int r = 0; r < nseg; ++r) total += cnt[r];
  Segs sg{base, cnt, cap, nseg};
  u64 T = 0;
  if (total >= (uint32_t)K) T = select_kth(sg, K, hist);
  if (p.tau_out != nullptr && lane == 0) p.tau_out[q] = (total >= (uint32_t)K) ? key_score(T) : -INFINITY;
  if (p.out_idx == nullptr) return;
  // Exactly min(K, total) entries are >= T; write them in region order.
  int32_t* oi = p.out_idx + (int64_t)q * K;
  float* os = p.out_score ? p.out_score + (int64_t)q * K : nullptr;
  uint32_t out = 0;
  for (int r = 0; r < nseg; ++r) {
    const u64* src = sg.ptr(r);
    const uint32_t n = cnt[r];
    for (uint32_t b0 = 0; b0 < n; b0 += 64) {
      const uint32_t i = b0 + lane;
      const u64 e = (i < n) ? src[i] : 0ull;
      const bool keep = (i < n) && (e >= T);
      const u64 m = __ballot(keep);
      const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
      if (keep && out + before < (uint32_t)K) {
        oi[out + before] = key_pos(e);
        if (os) os[out + before] = key_score(e);
      }
      out += __popcll(m);
    }
  }
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
  const int q = blockIdx.x;
  const int lane = lane_id();
  const int R = p.cb.R, cap = p.cb.cap, K = p.topk;
  const u64* base = p.cb.cand + ((int64_t)q * R + p.r0) * cap;
  const uint32_t* cnt = p.cb.counts + (int64_t)q * R + p.r0;
  const int nseg = p.r1 - p.r0;
  uint32_t total = 0;
  for (int r = 0; r < nseg; ++r) total += cnt[r];
  Segs sg{base, cnt, cap, nseg};
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
    const uint32_t n = cnt[r];
    for (uint32_t b0 = 0; b0 < n; b0 += 64) {
      const uint32_t i = b0 + lane;
      const u64 e = (i < n) ? src[i] : 0ull;
      const bool keep = (i < n) && (e >= T);
      const u64 m = __ballot(keep);
      const uint32_t before = __popcll(m & ((1ull << lane) - 1ull));
      if (keep && out + before < (uint32_t)K) keys[out + before] = e;
      out += __popcll(m);
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

template <int C, int H, int D>
static hipError_t launch_score_t(const ScoreLaunch& p, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  hipLaunchKernelGGL((score_kernel<C, H, D>), dim3(p.n_items), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int C>
static hipError_t dispatch_hd(int H, int d, const ScoreLaunch& p, hipStream_t s) {
#define DOSA_HD(HH, DD) \
  if (H == HH && d == DD) return launch_score_t<C, HH, DD>(p, s);
  DOSA_HD(8, 64) DOSA_HD(16, 64) DOSA_HD(32, 64) DOSA_HD(64, 64)
  DOSA_HD(8, 128) DOSA_HD(16, 128) DOSA_HD(32, 128) DOSA_HD(64, 128)
#undef DOSA_HD
  return hipErrorInvalidValue;
}

hipError_t launch_score(int combo, int H, int d, const ScoreLaunch& p, hipStream_t s) {
  switch (combo) {
    case C_F32: return dispatch_hd<C_F32>(H, d, p, s);
    case C_BF16: return dispatch_hd<C_BF16>(H, d, p, s);
    case C_FP8: return dispatch_hd<C_FP8>(H, d, p, s);
    case C_BF16Q_FP8K: return dispatch_hd<C_BF16Q_FP8K>(H, d, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectLaunch& p, hipStream_t s) {
  if (p.total_q == 0) return hipSuccess;
  if (p.sorted && p.out_idx != nullptr)
    hipLaunchKernelGGL(select_sorted_kernel, dim3(p.total_q), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(select_kernel, dim3(p.total_q), dim3(64), 0, s, p);
  return hipGetLastError();
}

bool combo_supported(int combo, int H, int d) {
  if (combo < 0 || combo > 3) return false;
  if (!(d == 64 || d == 128)) return false;
  if (!(H == 8 || H == 16 || H == 32 || H == 64)) return false;
  return true;
}

}  // namespace dosa

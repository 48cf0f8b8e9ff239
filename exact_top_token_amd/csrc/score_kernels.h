// Exact all-head scoring on MFMA with a streaming per-query candidate buffer.
//
// A wavefront scores a query group (QW consecutive queries of a sequence).
// MFMA rows are (query, head slot) pairs, columns are 16 keys, the reduction
// runs over the head dimension d:
//     x[(t,h), s] = q[t,h,:] . k[s,:]            (fp32 accumulation)
// and each lane folds its 4 output rows -- 4 heads of one query -- into the
// score through the identity w max(0,x) = w x/2 + w |x|/2:
//     S(t,s) = sum_h (w'_h/2) |x_h|  +  (q_scale/2) qbar_t . k_s   (then x k_scale)
// with w'_h = w_h x q_scale (the query's fp8 scale, 1 otherwise)
// with qbar_t = sum_h w_h q_h evaluated by one more MFMA row group (its terms
// come from prep.hip), so each head value costs one fused multiply-add with
// a free |.| operand modifier.  After all head groups every lane holds a
// finished score with no cross-lane reduction (QW = 4; QW = 2/1 need one/two
// lane exchanges).
//
// Two kernels share that arithmetic, so a (query, key) pair gets the same
// fp32 score whichever kernel computes it:
//   score_tiled_kernel  8 wavefronts (8 query groups) share key tiles staged
//                       through LDS, double-buffered with register prefetch;
//                       used for key ranges (dense path, seed pass).
//   score_list_kernel   one wavefront per query group walking a key range or a
//                       survivor list with its own loads (pruned path).
// Both carry a ROLE template argument (dense path, seed pass, survivor pass)
// that changes nothing in the code: each pass gets kernels of its own name,
// so profiles attribute time per pass.  Each operand combination's kernels
// are instantiated in a source file of their own (score_<combo>.hip).
//
// Scores at or above the query's running threshold theta are appended to the
// query's candidate region as packed (score, position) keys (DoSA pages,
// Method section: full scoring fused with threshold filtering, scores packed
// for selection; Related Work: radix selection, bounded-buffer streaming).
// theta comes from a per-query LDS histogram of the scores that reached
// theta: 256 bins of 1/32 octave on the order-preserving integer image of the
// float, anchored below the first block's maximum.  The lower edge of the
// highest bin with at least K counted scores at or above it never exceeds
// the K-th largest score seen, so it is a valid filter at all times (scores
// below theta are left out: they can only lie in bins at or below theta's,
// so leaving them out can delay a raise but never make one wrong).  A full region is
// compacted at theta in one pass; only if that frees too little does the
// wavefront run an exact radix select.
#pragma once
#include "dosa_device.h"

namespace dosa {

constexpr int kTileKeys = 64;   // keys per LDS tile


// K-th largest of the n distinct entries at ptr, by one wavefront with a
// private 256-bin LDS histogram (8-bit digits from the top; no workgroup
// barrier, so the other wavefronts keep working).  Returns T with exactly K
// entries >= T.
__device__ __noinline__ u64 select_kth_wave(const u64* ptr, uint32_t n, int K, uint32_t* hist) {
  const int lane = lane_id();
  u64 prefix = 0;
  uint32_t rem = (uint32_t)K;
  wave_sync();
#pragma unroll 1
  for (int p = 0; p < 8; ++p) {
    const int sh = 56 - 8 * p;
    const int hs = sh + 8;
    for (int b = lane; b < 256; b += 64) hist[b] = 0;
    wave_sync();
    const u64 want = (p == 0) ? 0 : (prefix >> hs);
    for (uint32_t b = 0; b < n; b += 64 * kBatch) {
      u64 e[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = b + 64u * u + lane;
        e[u] = (i < n) ? ptr[i] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = b + 64u * u + lane;
        if (i < n && (p == 0 || (e[u] >> hs) == want)) atomicAdd(&hist[(uint32_t)(e[u] >> sh) & 255u], 1u);
      }
    }
    wave_sync();
    uint32_t s = 0;
    for (int t = 0; t < 4; ++t) s += hist[lane * 4 + t];
    const uint32_t suf = wave_suffix_sum(s);
    const bool cross = (suf >= rem) && (suf - s < rem);
    const u64 cm = __ballot(cross);
    const int L = cm ? (__ffsll((long long)cm) - 1) : 0;
    uint32_t acc = __shfl(suf - s, L, 64);
    int b = L * 4;
    uint32_t cnt_b = 0;
    for (int t = 3; t >= 0; --t) {
      const uint32_t h = hist[L * 4 + t];
      if (acc + h >= rem) { b = L * 4 + t; cnt_b = h; break; }
      acc += h;
    }
    rem -= acc;
    prefix |= ((u64)(uint32_t)b) << sh;
    wave_sync();
    if (cnt_b == rem) break;
  }
  return prefix;
}

// Region compaction for the streaming select: keep the entries >= tq of
// the n at bq; if more than half the region is still in use, select the
// exact K-th and keep K.  Returns the new count in the low 31 bits, bit 31
// set if a select ran, and the new threshold's bits in the high word.
__device__ __noinline__ u64 shrink_region(u64* bq, uint32_t n, float tq, int cap, int K, uint32_t* shist) {
  uint32_t nk = n;
  float th = tq;
  uint32_t sel = 0;
  if (tq > -INFINITY) {
    nk = compact_ge(bq, n, (u64)f2ord(tq) << 32, bq, 0);
    wave_sync();
  }
  if (nk > (uint32_t)(cap / 2) && nk > (uint32_t)K) {
    const u64 T = select_kth_wave(bq, nk, K, shist);
    compact_ge(bq, nk, T, bq, 0);
    wave_sync();
    nk = (uint32_t)K;
    th = fmaxf(th, key_score(T));
    sel = 1u;
  }
  return ((u64)__float_as_uint(th) << 32) | (u64)(nk | (sel << 31));
}

constexpr int kHistBins = 256;          // running-threshold histogram bins per query
constexpr int kHistShift = 18;          // 2^18 ord units per bin: 32 bins per octave
constexpr int kHistAnchor = 192;        // the first block's maximum lands in this bin
// 64-key tiles between two threshold refreshes of the tiled kernel.  A
// refresh costs about as much as appending a tile's candidates; every 16
// tiles measured fastest (8 appends 3% fewer candidates and runs slower).
constexpr int kRefreshTiles = 16;

template <int C, int H, int D>
struct Scorer {
  using O = Ops<C, D>;
  static constexpr int QW = queries_per_wave(C, H, D);
  static constexpr int S = 16 / QW;   // head slots per query in one MFMA
  static constexpr int HG = H / S;    // head groups
  static constexpr int STEPS = O::STEPS;
  static constexpr int KBYTES = D * O::KB;

  typename O::frag A[HG][STEPS];
  typename O::frag AL[STEPS];       // weighted-query terms of the group's queries
  int q_row0, pos0, nq;   // the group's first query row and position, its query count (wavefront-uniform)
  // Lane roles, recomputed from the lane id where used (cheaper than holding
  // them in registers across the scoring loop).
  __device__ __forceinline__ int col() const { return lane_fresh() & 15; }
  __device__ __forceinline__ int g() const { return lane_fresh() >> 4; }
  __device__ __forceinline__ int qi() const { return (4 * g()) / S; }
  __device__ __forceinline__ int qrow() const { return q_row0 + qi(); }
  __device__ __forceinline__ int pos() const { return pos0 + qi(); }
  __device__ __forceinline__ int owner_lane0() const { return 16 * (qi() * (4 / QW)); }
  __device__ __forceinline__ bool qok() const { return qi() < nq; }
  __device__ __forceinline__ bool owner() const { return g() == (owner_lane0() >> 4); }
  float theta;
  uint32_t count;
  u64* buf;
  uint32_t wq_lds;   // LDS byte address of this lane's query's weights / 2, then its term scales / 2
  uint32_t* qh;      // LDS: this wavefront's query histograms [QW][kHistBins]
  uint32_t hbase;    // ord value of the lower edge of bin 0 (0 = not anchored yet)
  uint32_t* tshare;  // the call's shared thresholds (indexed by query row), or NULL
  uint32_t* anchor;  // LDS [QW]: histogram anchors shared with the workgroup's other wavefronts, or NULL
  uint32_t* tpart;   // the call's split thresholds (ScoreLaunch::theta_part) at this sweep's query rows, or NULL
  int part_stride, part_n, part_idx;
  uint32_t n_written, n_reselect, n_scored;
  bool dirty;        // something was appended since the last refresh (wavefront-uniform)

  // wl: LDS [QW][H + S]: per query the head weights / 2, then the scales / 2
  // of its weighted-query terms (filled here);
  // hq: LDS [QW][kHistBins] running-threshold histograms (zeroed here).
  __device__ __forceinline__ void init(const ScoreLaunch& p, const GroupInfo& gr, int region, float* wl,
                                       uint32_t* hq, bool active, bool write_lds = true) {
    const int lane = lane_id(), g = lane >> 4;
    nq = active ? gr.nq : 0;
    q_row0 = gr.q_row0;
    pos0 = gr.pos0;
    {
      const int ra = lane & 15;
      const int qa = ra / S, hs = ra % S;
      const bool ok = qa < nq;
      const uint8_t* qb = static_cast<const uint8_t*>(p.in.q);
      const int Hr = p.in.H;   // heads stored per query row (head slots past it stay zero)
#pragma unroll
      for (int j = 0; j < HG; ++j) {
        const int head = S * j + hs;
        if (ok && (H == Hr || head < Hr))
          O::load_q(qb + ((int64_t)(gr.q_row0 + qa) * Hr + head) * D * O::QB, g, A[j]);
        else
          O::zero(A[j]);
      }
      if (ok)
        O::load_q(static_cast<const uint8_t*>(p.lrows) + ((int64_t)(gr.q_row0 + qa) * S + hs) * D * O::QB, g, AL);
      else
        O::zero(AL);
    }
    // the query's fp8 scale is folded into its weights here, so a score is
    // (sum of weighted terms) x key scale with no per-score query-scale product
    for (int e = lane; write_lds && e < QW * (H + S); e += 64) {
      const int q = e / (H + S), h = e % (H + S);
      float v = 0.f;
      if (q < nq) {
        const float qsc = HasQScale<C>::value ? p.in.q_scale[gr.q_row0 + q] : 1.f;
        if (h >= H) v = (0.5f * p.lsig[(int64_t)(gr.q_row0 + q) * S + (h - H)]) * qsc;
        else if (h < p.in.H) v = (0.5f * p.in.w[(int64_t)(gr.q_row0 + q) * p.in.H + h]) * qsc;
      }
      wl[e] = v;
    }
    wq_lds = (uint32_t)(uintptr_t)(wl + qi() * (H + S));   // low 32 bits of a generic LDS address = the LDS offset
    // lanes of absent queries get an unreachable threshold, so they never append
    theta = qok() ? (p.theta_init != nullptr ? p.theta_init[qrow()] : -INFINITY) : INFINITY;
    count = 0;
    buf = qok() ? p.cb.row(qrow(), region) : nullptr;
    qh = hq;
    if (write_lds)
      for (int e = lane; e < QW * kHistBins; e += 64) hq[e] = 0;
    hbase = 0;
    anchor = nullptr;
    tshare = p.theta_share;
    tpart = nullptr;
    part_stride = p.part_stride;
    part_n = 0;
    part_idx = 0;
    n_written = n_reselect = n_scored = 0;
    dirty = false;
  }

  // The item's place among the launch's sweeps over its queries' keys (split
  // thresholds, ScoreLaunch::theta_part); off with one sweep.
  __device__ __forceinline__ void set_part(const ScoreLaunch& p, const WorkItem& it) {
    if (p.theta_part != nullptr && it.nparts > 1) {
      tpart = p.theta_part + p.part_base;
      part_n = it.nparts;
      part_idx = it.region - p.part_rbase;
    }
  }

  // Raise theta of every query of the wavefront to the lower edge of the
  // highest histogram bin that has at least K scores at or above it.  The
  // queries are handled side by side: each owns 64/QW lanes, each lane 4*QW
  // consecutive bins; a segmented suffix sum over the query's lanes finds the
  // lane whose bins hold the K-th count, which walks its own bins.
  __device__ __forceinline__ void refresh_theta(int K) {
    constexpr int LPQ = 64 / QW;                 // lanes per query
    constexpr int BPL = kHistBins / LPQ;         // bins per lane
    wave_sync();
    const int ln = lane_fresh();
    const int j = ln % LPQ, q = ln / LPQ;        // q == qi()
    if (anchor != nullptr && hbase == 0u) hbase = anchor[q];   // anchored by another wavefront
    const uint32_t* h = qh + q * kHistBins + j * BPL;
    uint32_t hv[BPL];
#pragma unroll
    for (int t = 0; t < BPL; t += 4) {
      const v4i v = *reinterpret_cast<const v4i*>(h + t);
      hv[t] = (uint32_t)v[0]; hv[t + 1] = (uint32_t)v[1]; hv[t + 2] = (uint32_t)v[2]; hv[t + 3] = (uint32_t)v[3];
    }
    uint32_t s = 0;
#pragma unroll
    for (int t = 0; t < BPL; ++t) s += hv[t];
    uint32_t suf = s;
#pragma unroll
    for (int off = 1; off < LPQ; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_down((int)suf, off, LPQ);
      if (j + off < LPQ) suf += o;
    }
    const bool cross = hbase != 0u && suf >= (uint32_t)K && suf - s < (uint32_t)K;
    uint32_t a = suf - s;
    int bt = 0;
    bool found = false;
#pragma unroll
    for (int t = BPL - 1; t >= 0; --t) {
      const bool hit = !found && a + hv[t] >= (uint32_t)K;
      bt = hit ? t : bt;
      found = found || hit;
      a += hv[t];
    }
    uint32_t edge = hbase + ((uint32_t)(j * BPL + bt) << kHistShift);
    if (edge < hbase || edge > 0xFF7FFFFFu) edge = 0xFF7FFFFFu;   // stay on finite floats
    const u64 cm = __ballot(cross);
    const u64 segm = (cm >> (q * LPQ)) & (LPQ == 64 ? ~0ull : ((1ull << (LPQ & 63)) - 1ull));
    const int L = segm ? q * LPQ + (__ffsll((long long)segm) - 1) : ln;
    const uint32_t e = (uint32_t)__shfl((int)edge, L, 64);
    if (segm != 0ull) {
      const float th = ord2f(e);
      if (th > theta) theta = th;
    }
    if (tpart != nullptr) {
      // This sweep's ceil(K / part_n)-th largest score so far (the lower
      // edge of its bin), published for the launch's part_n disjoint sweeps
      // over the query's keys.  Each published value has that many of its
      // sweep's scores at or above it, so the smallest of all part_n values
      // has at least K scores at or above it among the query's keys: a valid
      // threshold, near the K-th largest of all the sweeps' scores together,
      // where each sweep's own histogram reaches only its own K-th.
      const uint32_t K2 = ((uint32_t)K + (uint32_t)part_n - 1u) / (uint32_t)part_n;
      const bool cross2 = hbase != 0u && suf >= K2 && suf - s < K2;
      uint32_t a2 = suf - s;
      int bt2 = 0;
      bool found2 = false;
#pragma unroll
      for (int t = BPL - 1; t >= 0; --t) {
        const bool hit = !found2 && a2 + hv[t] >= K2;
        bt2 = hit ? t : bt2;
        found2 = found2 || hit;
        a2 += hv[t];
      }
      uint32_t edge2 = hbase + ((uint32_t)(j * BPL + bt2) << kHistShift);
      if (edge2 < hbase || edge2 > 0xFF7FFFFFu) edge2 = 0xFF7FFFFFu;
      const u64 cm2 = __ballot(cross2);
      const u64 segm2 = (cm2 >> (q * LPQ)) & (LPQ == 64 ? ~0ull : ((1ull << (LPQ & 63)) - 1ull));
      const int L2 = segm2 ? q * LPQ + (__ffsll((long long)segm2) - 1) : ln;
      const uint32_t e2 = (uint32_t)__shfl((int)edge2, L2, 64);
      uint32_t* row = tpart + (int64_t)(q_row0 + q) * part_stride;
      if (segm2 != 0ull && j == 0 && q < nq) atomicMax(row + part_idx, e2);
      uint32_t mn = 0xFFFFFFFFu;
      for (int r = j; r < part_n; r += LPQ)
        mn = min(mn, q < nq ? __hip_atomic_load(row + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u);
#pragma unroll
      for (int off = 1; off < LPQ; off <<= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, LPQ));
      if (q < nq && mn != 0u && mn != 0xFFFFFFFFu) theta = fmaxf(theta, ord2f(mn));
    }
    // Share with the call's other sweeps over this query's keys: publish the
    // threshold and adopt the largest one published.  Any sweep's threshold
    // is at most the K-th largest score among its own keys, hence at most the
    // query's K-th largest, so filtering by it never drops a Top-K key.
    if (tshare != nullptr) {
      uint32_t gv = 0u;
      if (j == 0 && q < nq) gv = atomicMax(tshare + q_row0 + q, f2ord(theta));
      gv = (uint32_t)__shfl((int)gv, q * LPQ, 64);
      if (gv != 0u && q < nq) theta = fmaxf(theta, ord2f(gv));
    }
    dirty = false;
  }

  // Compact the region of query qq to the entries >= its theta; if that
  // leaves it more than half full, select the exact K-th and keep K.  The
  // work is a call (shrink_region), so its registers do not weigh on the
  // scoring loop around it.
  __device__ __forceinline__ void shrink(const ScoreLaunch& p, const GroupInfo& gr, int region, int qq,
                                         uint32_t* shist) {
    const int cap = p.cb.cap;
    const uint32_t cq = __shfl(count, 16 * (qq * (4 / QW)), 64);
    const float tq = __shfl(theta, 16 * (qq * (4 / QW)), 64);
    u64* bq = p.cb.row(gr.q_row0 + qq, region);
    const u64 r = shrink_region(bq, cq, tq, cap, p.topk, shist);
    const uint32_t nk = (uint32_t)r & 0x7FFFFFFFu;
    if ((uint32_t)r >> 31) ++n_reselect;
    if (qi() == qq) {
      count = nk;
      theta = __uint_as_float((uint32_t)(r >> 32));
    }
  }

  __device__ __forceinline__ static v4f mma_all(const typename O::frag* a, const typename O::frag* B) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s) c = O::mma(a[s], B[s], c);
    return c;
  }

  // Unscaled scores of this lane's (query, key column) for NB 16-key blocks
  // whose fragments are in B[0..NB).  Head groups run in the outer loop, so
  // one LDS read of a group's weights serves all NB blocks and the NB MFMAs
  // of a group are independent of each other.  A block's value is the same
  // sequence of operations whatever NB is, so a (query, key) score does not
  // depend on which kernel computes it or on the other keys of the step.
  template <int NB>
  __device__ __forceinline__ void scoreN(const typename O::frag (*Bin)[STEPS], float* out) const {
    // Software pipeline pinned with empty volatile asm statements (which the
    // compiler keeps in program order): iteration j issues the MFMAs of head
    // group j+1 -- their key fragments are re-versioned at the start of the
    // iteration so they cannot be hoisted earlier -- then folds group j, whose
    // MFMAs were issued one iteration before; the accumulators are pinned at
    // the end of the iteration so the FMAs cannot sink later.
    typename O::frag B[NB][STEPS];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) B[b][s] = Bin[b][s];
    float o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = 0.f;
    uint32_t wa = wq_lds + 4u * (uint32_t)((4 * g()) % S);
    asm volatile("" : "+v"(wa));
    typedef __attribute__((address_space(3))) const v4f lds_v4f;
    v4f cur[NB];
    // Wave priority (s_setprio, inside this wavefront only): 2 while a burst
    // of MFMAs issues, 1 for the rest of the scoring, 0 outside it.  When the
    // two wavefronts of a SIMD compete, the one about to feed the matrix pipe
    // issues first and the one appending candidates fills the gaps (3% faster
    // on MI355X than equal priorities).
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int b = 0; b < NB; ++b) cur[b] = mma_all(A[0], B[b]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < HG; ++j) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < STEPS; ++s) asm volatile("" : "+v"(B[b][s]));
      const v4f w4 = *reinterpret_cast<lds_v4f*>((uintptr_t)(wa + 4u * (uint32_t)(S * j)));
      v4f nxt[NB];
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int b = 0; b < NB; ++b) nxt[b] = (j + 1 < HG) ? mma_all(A[j + 1 < HG ? j + 1 : 0], B[b]) : mma_all(AL, B[b]);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        o[b] = fmaf(w4[0], fabsf(cur[b][0]), o[b]);
        o[b] = fmaf(w4[1], fabsf(cur[b][1]), o[b]);
        o[b] = fmaf(w4[2], fabsf(cur[b][2]), o[b]);
        o[b] = fmaf(w4[3], fabsf(cur[b][3]), o[b]);
        asm volatile("" : "+v"(o[b]));
        cur[b] = nxt[b];
      }
    }
    const v4f sl = *reinterpret_cast<lds_v4f*>((uintptr_t)(wa + 4u * (uint32_t)(S * HG)));
    __builtin_amdgcn_s_setprio(0);   // no MFMA left to issue
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[b] = fmaf(sl[i], cur[b][i], o[b]);
      if constexpr (QW <= 2) o[b] += __shfl_xor(o[b], 16, 64);
      if constexpr (QW == 1) o[b] += __shfl_xor(o[b], 32, 64);
      out[b] = o[b];
    }
  }

  // Count the scores of one step (4 blocks of 16 keys) in their queries'
  // histograms, append those that reach theta, and shrink regions that are
  // about to overflow.  Called by all 64 lanes of the wavefront.  CHECK: some
  // keys of the step may lie outside the range (kvalid) or after a query's
  // position; without it every key of the step is visible to every query of
  // the group.  KBASE: the step's keys are kbase + 16 b + column (a key range),
  // computed only when a score is taken; otherwise they come in key[].  Lanes
  // of absent queries hold theta = +inf and never take.  A step whose scores
  // all stay below theta costs a few instructions.  A step adds at most 64
  // entries per query, so regions are checked against cap - 64 once per step.
  template <bool CHECK, bool KBASE = false>
  __device__ __forceinline__ void append4(const ScoreLaunch& p, const GroupInfo& gr, int region, const float* o,
                                          const float* ks, const int* key, const bool* kvalid, uint32_t* shist,
                                          int kbase = 0) {
    float sc[4];
    bool take[4];
    bool anyt = false;
    if constexpr (CHECK || QW < 4) {
      const int gg = lane_fresh() >> 4;
      const int q_i = (4 * gg) / S;
      const bool own = (QW == 4) || (gg == ((16 * (q_i * (4 / QW))) >> 4));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sc[b] = o[b] * ks[b];
        bool v = own;
        if constexpr (CHECK) {
          v = v && kvalid[b] && key[b] <= pos0 + q_i && q_i < nq;
          n_scored += __popcll(ballot(v));
        }
        take[b] = v && sc[b] >= theta;
        anyt = anyt || take[b];
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sc[b] = o[b] * ks[b];
        take[b] = sc[b] >= theta;
        anyt = anyt || take[b];
      }
    }
    if constexpr (!CHECK) n_scored += 64u * (uint32_t)nq;
    if (ballot(anyt) == 0ull) return;
    dirty = true;
    const int ln = lane_fresh();
    const int c = ln & 15, gg = ln >> 4;
    const int q_i = (4 * gg) / S;
    const int ol0 = 16 * (q_i * (4 / QW));
    uint32_t so[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) so[b] = f2ord(sc[b]);
    if (ballot(hbase == 0) != 0ull) {
      // anchor each query's histogram below the maximum of the first scores
      // it takes (all lanes take part in the exchanges; only unanchored
      // queries update)
      uint32_t mx = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) mx = max(mx, take[b] ? so[b] : 0u);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
      mx = __shfl(mx, ol0 + c, 64);
      if (hbase == 0 && mx != 0u) {
        const uint32_t lo = (uint32_t)kHistAnchor << kHistShift;
        uint32_t a = (mx > 0x00800000u + lo) ? mx - lo : 0x00800000u;
        if (anchor != nullptr) {
          // one anchor per query for the workgroup: the first wavefront to take sets it
          const uint32_t prev = atomicCAS(&anchor[q_i], 0u, a);
          a = prev != 0u ? prev : a;
        }
        hbase = a;
      }
    }
    uint32_t* hq = qh + q_i * kHistBins;
    const uint32_t below = (1u << c) - 1u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const u64 m = ballot(take[b]);
      if (m == 0ull) continue;
      if (take[b] && hbase != 0 && so[b] >= hbase)
        atomicAdd(&hq[min((so[b] - hbase) >> kHistShift, (uint32_t)(kHistBins - 1))], 1u);
      const uint32_t slice = (uint32_t)(m >> ol0) & 0xFFFFu;
      if (take[b]) {
        const int kk = KBASE ? kbase + 16 * b + c : key[b];
        buf[count + __popc(slice & below)] = ((u64)so[b] << 32) | (u64)(uint32_t)(~(uint32_t)kk);
      }
      count += __popc(slice);
      n_written += __popcll(m);
    }
    const uint32_t hi_water = (uint32_t)(p.cb.cap - 64);
    if (ballot(count > hi_water) != 0ull) {
      refresh_theta(p.topk);
#pragma unroll 1
      for (int qq = 0; qq < QW; ++qq)
        if (__shfl(count, 16 * (qq * (4 / QW)), 64) > hi_water) shrink(p, gr, region, qq, shist);
    }
  }


  // End of the sweep: bring every region down to its final theta.
  // Every region is cut, also one holding fewer than K entries: with many
  // regions per query (a split kernel's eight wavefronts times its key
  // splits) the final merge would otherwise read every appended candidate
  // in each of its passes.
  __device__ __forceinline__ void close(const ScoreLaunch& p, const GroupInfo& gr, int region, uint32_t* shist) {
    refresh_theta(p.topk);
#pragma unroll 1
    for (int qq = 0; qq < QW; ++qq) {
      const uint32_t cq = __shfl(count, 16 * (qq * (4 / QW)), 64);
      const float tq = __shfl(theta, 16 * (qq * (4 / QW)), 64);
      if (cq > 0u && tq > -INFINITY) {
        u64* bq = p.cb.row(gr.q_row0 + qq, region);
        const uint32_t nk = compact_ge(bq, cq, (u64)f2ord(tq) << 32, bq, 0);
        if (qi() == qq) count = nk;
      }
    }
    wave_sync();
  }

  __device__ __forceinline__ void finish(const ScoreLaunch& p, int region) {
    if (qok() && lane_id() == owner_lane0()) *p.cb.count(qrow(), region) = count;
    if (p.stats != nullptr && lane_id() == 0) {
      atomicAdd(&p.stats[p.scored_slot], (u64)n_scored);
      if (p.scored_slot2 > 0) atomicAdd(&p.stats[p.scored_slot2], (u64)n_scored);
      atomicAdd(&p.stats[5], (u64)n_written);
      atomicAdd(&p.stats[6], (u64)n_reselect);
    }
  }
};

// ---------------------------------------------------------------------------
// one wavefront per query group: key range (two sub-ranges walked top-down)
// or survivor list (ascending)
// ---------------------------------------------------------------------------
// fp8 keys leave room for two wavefronts per SIMD, which hides the
// latency of the per-step key gather; the wider f32/bf16 rows would spill.
template <int C, int H, int D, int ROLE>
__global__ __launch_bounds__(64, KeyRaw<C>::value ? 2 : 1) void score_list_kernel(const ScoreLaunch p) {
  using SC = Scorer<C, H, D>;
  using O = typename SC::O;
  __shared__ uint32_t hist[256];
  __shared__ __attribute__((aligned(16))) float wl[SC::QW * (H + SC::S)];
  __shared__ uint32_t qhist[SC::QW * kHistBins];
  if (skip_launch(p.mode, p.run_if)) return;
  const WorkItem it = p.items[blockIdx.x];
  const GroupInfo gr = p.groups[it.group];
  if (p.flag_mode != 0) {
    bool all = true;
    for (int i = 0; i < gr.tile_n; ++i) all = all && (p.tile_flags[gr.tile_first + i] != 0);
    if (p.flag_mode == 2 && all) return;    // this tile's bounded range is scored whole
    if (p.flag_mode == 1 && !all) return;   // this group's survivor list is scored instead
  }
  SC sc;
  sc.init(p, gr, it.region, wl, qhist, true);
  __syncthreads();
  int nblk = 0;
  const uint8_t* kbytes = static_cast<const uint8_t*>(p.in.k);

  auto load = [&](int key, bool kvalid, typename O::frag* B, float& ks) {
    ks = 1.f;
    if (kvalid) {
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      O::load_k(kbytes + row * SC::KBYTES, sc.g(), B);
      if constexpr (HasKScale<C>::value) ks = p.in.k_scale[row];
    } else {
      O::zero(B);
    }
  };
  // four 16-key blocks per step
  auto step4 = [&](const int* keys, const bool* v) {
    float ks[4], o[4];
    if constexpr (KeyRaw<C>::value) {
      // two blocks of fragments at a time (the register budget of the
      // prefetching range walk above)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        typename O::frag B[2][SC::STEPS];
#pragma unroll
        for (int b = 0; b < 2; ++b) load(keys[2 * j + b], v[2 * j + b], B[b], ks[2 * j + b]);
        sc.template scoreN<2>(B, o + 2 * j);
      }
    } else {
      typename O::frag B[4][SC::STEPS];
#pragma unroll
      for (int b = 0; b < 4; ++b) load(keys[b], v[b], B[b], ks[b]);
      sc.template scoreN<4>(B, o);
    }
    sc.template append4<true>(p, gr, it.region, o, ks, keys, v, hist);
    if ((++nblk & 7) == 0 && sc.dirty) sc.refresh_theta(p.topk);
  };

  if constexpr (KeyRaw<C>::value) {
    if (!it.gather) {
      // The range walk with the next step's key bytes on their way while the
      // current step is scored: one wavefront works alone on its keys, so
      // without this every step waits out a full memory latency.
      const int na = it.a1 > it.a0 ? (it.a1 - it.a0 + 63) / 64 : 0;
      const int ns = na + (it.b1 > it.b0 ? (it.b1 - it.b0 + 63) / 64 : 0);
      auto step_kb = [&](int s, int& lo, int& hi) -> int {
        const bool ra = s < na;
        lo = ra ? it.a0 : it.b0;
        hi = ra ? it.a1 : it.b1;
        return hi - 16 - 64 * (ra ? s : s - na);
      };
      // Half steps of two 16-key blocks: the raw bytes of the next half are
      // in flight while the current one is scored (two blocks of fragments
      // at a time keep the kernel within two wavefronts per SIMD); the four
      // blocks of a step are appended together.
      typename O::raw rn[2];
      float ksn[2];
      auto fetch = [&](int h) {
        int lo, hi;
        const int kb = step_kb(h >> 1, lo, hi) - 32 * (h & 1);
        const int cl = sc.col();
        // rows first (page-table reads of both blocks in flight together),
        // then the key bytes and scales
        int64_t row[2];
        bool ok[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int key = kb - 16 * b + cl;
          ok[b] = key >= lo && key < hi;
          row[b] = ok[b] ? key_row(p.in, gr.key_base, gr.seq, key) : 0;
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          ksn[b] = 1.f;
          if (ok[b]) {
            O::load_raw(kbytes + row[b] * SC::KBYTES, sc.g(), rn[b]);
            if constexpr (HasKScale<C>::value) ksn[b] = p.in.k_scale[row[b]];
          } else {
            rn[b] = typename O::raw{};
          }
        }
      };
      if (ns > 0) fetch(0);
#pragma unroll 1
      for (int s = 0; s < ns; ++s) {
        int lo, hi;
        const int kb = step_kb(s, lo, hi);
        int keys[4];
        bool v[4];
        float ks[4], o[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          keys[b] = kb - 16 * b + sc.col();
          v[b] = keys[b] >= lo && keys[b] < hi;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          typename O::frag B[2][SC::STEPS];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            O::from_raw(rn[b], B[b]);
            ks[2 * j + b] = ksn[b];
          }
          if (2 * s + j + 1 < 2 * ns) fetch(2 * s + j + 1);
          sc.template scoreN<2>(B, o + 2 * j);
        }
        sc.template append4<true>(p, gr, it.region, o, ks, keys, v, hist);
        if ((++nblk & 7) == 0 && sc.dirty) sc.refresh_theta(p.topk);
      }
      sc.close(p, gr, it.region, hist);
      sc.finish(p, it.region);
      return;
    }
  }
  if (!it.gather) {
#pragma unroll 1
    for (int r = 0; r < 2; ++r) {
      const int lo = r ? it.b0 : it.a0, hi = r ? it.b1 : it.a1;
#pragma unroll 1
      for (int kb = hi - 16; kb > lo - 16; kb -= 64) {
        int keys[4];
        bool v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          keys[b] = kb - 16 * b + sc.col();
          v[b] = keys[b] >= lo && keys[b] < hi;
        }
        step4(keys, v);
      }
    }
  } else {
    const int32_t* lst = p.list_stride > 0 ? p.lists + (int64_t)it.group * p.list_stride
                                           : p.lists + gr.list_off + (p.list_start != nullptr ? p.list_start[it.group] : 0);
    const int len = p.list_len[it.group];
    const int e0 = (int)(((int64_t)len * it.a0 / it.a1) & ~15LL);
    const int e1 = (it.a0 == it.a1 - 1) ? len : (int)(((int64_t)len * (it.a0 + 1) / it.a1) & ~15LL);
#pragma unroll 1
    for (int e = e0; e < e1; e += 64) {
      int keys[4];
      bool v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i0 = e + 16 * b + sc.col();
        v[b] = i0 < e1;
        keys[b] = v[b] ? lst[i0] : 0;
      }
      step4(keys, v);
    }
  }
  sc.close(p, gr, it.region, hist);
  sc.finish(p, it.region);
}

// ---------------------------------------------------------------------------
// Decode-like batches (query tiles of fewer than 4 groups): the 8 wavefronts
// of a workgroup score ONE query group over the item's key range (or its
// share of the group's survivor list), taking the 64-key steps round robin:
// wavefront w scores steps w, w + 8, w + 16, ...  Each wavefront appends to a
// region of its own (region r * 8 + w), but the running threshold of each
// query comes from one LDS histogram that all 8 wavefronts count into (one
// anchor per query, set by the first wavefront that takes a score), so it
// rises with every key the workgroup has scored instead of one wavefront's
// eighth of them; a workgroup also keeps 8 wavefronts' key loads in flight
// for one group, where one wavefront per group kept a single step's.
// ---------------------------------------------------------------------------
template <int C, int H, int D, int ROLE>
__global__ __launch_bounds__(64 * kTileWaves) void score_split_kernel(const ScoreLaunch p) {
  using SC = Scorer<C, H, D>;
  using O = typename SC::O;
  __shared__ uint32_t hist[kTileWaves][256];
  __shared__ __attribute__((aligned(16))) float wl[SC::QW * (H + SC::S)];
  __shared__ uint32_t qhist[SC::QW * kHistBins];
  __shared__ uint32_t anchor[SC::QW];
  // fp8 key rows of each wavefront's next step, streamed straight into LDS:
  // two images per wavefront (even and odd steps, separate arrays so the
  // compiler can tell a step's reads from the next step's stores)
  constexpr int KIMG = KeyRaw<C>::value ? kTileWaves * 64 * SC::KBYTES : 16;
  constexpr int SIMG = KeyRaw<C>::value ? kTileWaves * 64 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t kimg0[KIMG];
  __shared__ __attribute__((aligned(16))) uint8_t kimg1[KIMG];
  __shared__ float simg0[SIMG];
  __shared__ float simg1[SIMG];
  __shared__ __attribute__((aligned(16))) v4f opend[KeyRaw<C>::value ? kTileWaves * 64 : 1];   // a step's scores, appended in the next
  if (skip_launch(p.mode, p.run_if)) return;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x) >> 6;   // wavefront-uniform
  const WorkItem it = p.items[blockIdx.x];
  const GroupInfo gr = p.groups[it.group];
  if (p.flag_mode != 0) {
    bool all = true;
    for (int i = 0; i < gr.tile_n; ++i) all = all && (p.tile_flags[gr.tile_first + i] != 0);
    if (p.flag_mode == 2 && all) return;    // this tile's bounded range is scored whole
    if (p.flag_mode == 1 && !all) return;   // this group's survivor list is scored instead
  }
  SC sc;
  sc.init(p, gr, it.region * kTileWaves + wave, wl, qhist, true, wave == 0);
  sc.set_part(p, it);
  if (threadIdx.x < (unsigned)SC::QW) anchor[threadIdx.x] = 0u;
  sc.anchor = anchor;
  __syncthreads();
  int nstep = 0;
  uint32_t* shist = hist[wave];
  const uint8_t* kbytes = static_cast<const uint8_t*>(p.in.k);
  auto after_step = [&]() {
    // steps 2 and 3 of this wavefront, then every 4: the histogram also holds
    // the others' counts (the early refreshes raise the threshold from -inf
    // once the workgroup's first steps are counted)
    ++nstep;
    if ((nstep & 3) == 0 || nstep == 2 || nstep == 3) sc.refresh_theta(p.topk);
  };
  auto load = [&](int key, bool kvalid, typename O::frag* B, float& ks) {
    ks = 1.f;
    if (kvalid) {
      const int64_t row = key_row(p.in, gr.key_base, gr.seq, key);
      O::load_k(kbytes + row * SC::KBYTES, sc.g(), B);
      if constexpr (HasKScale<C>::value) ks = p.in.k_scale[row];
    } else {
      O::zero(B);
    }
  };
  // blocks of key fragments held at once: within the two-wavefronts-per-SIMD
  // register budget next to the query fragments
  constexpr int NBS = (int)sizeof(typename O::frag) * SC::STEPS <= 64 ? 2 : 1;
  auto step4 = [&](const int* keys, const bool* v) {
    float ks[4], o[4];
#pragma unroll
    for (int j = 0; j < 4 / NBS; ++j) {
      typename O::frag B[NBS][SC::STEPS];
#pragma unroll
      for (int b = 0; b < NBS; ++b) load(keys[NBS * j + b], v[NBS * j + b], B[b], ks[NBS * j + b]);
      sc.template scoreN<NBS>(B, o + NBS * j);
    }
    sc.template append4<true>(p, gr, it.region * kTileWaves + wave, o, ks, keys, v, shist);
    after_step();
  };
  const int region = it.region * kTileWaves + wave;

  if constexpr (KeyRaw<C>::value) {
    if (!it.gather && (p.in.page_table == nullptr || p.in.page_shift >= 6)) {
      // Range walk with the next step's 64 key rows and scales streamed by
      // direct global->LDS loads into this wavefront's own image while the
      // current step is scored: a step's key bytes (8 KiB at d = 128) are in
      // flight per wavefront without holding registers, and no barrier is
      // needed (each wavefront reads only the rows it loaded).  Image layout:
      // 16-byte unit u = 64 i + lane of load instruction i holds chunk
      // (u % CPK) ^ (r % CPK) of the step's key r = u / CPK, so the 16 lanes
      // that read one chunk column of 16 rows hit different banks.
      constexpr int KBY = SC::KBYTES;               // bytes per key row
      constexpr int CPK = KBY / 16;                 // 16-byte chunks per row (= load instructions per step)
      // Steps are the 64-key blocks of absolute key positions that meet the
      // range, from the top down: a step lies in one page (pages hold a
      // power of two >= 64 keys) and its rows are consecutive.
      auto nsteps = [](int lo, int hi) { return hi > lo ? (((hi + 63) & ~63) - (lo & ~63)) / 64 : 0; };
      const int na = nsteps(it.a0, it.a1);
      const int ns = na + nsteps(it.b0, it.b1);
      // step s: keys [base, base + 64), those in [lo, hi) valid
      auto step_base = [&](int s, int& lo, int& hi) -> int {
        const bool ra = s < na;
        lo = ra ? it.a0 : it.b0;
        hi = ra ? it.a1 : it.b1;
        return ((hi + 63) & ~63) - 64 - 64 * (ra ? s : s - na);
      };
      const bool paged = p.in.page_table != nullptr;
      const int sh = paged ? p.in.page_shift : 0;
      // the page table is read-only here: read through the constant address
      // space, so its wavefront-uniform entries come by scalar loads whose
      // waits the compiler places where they are used
      typedef __attribute__((address_space(4))) const int32_t cint;
      cint* ptab = paged ? (cint*)(p.in.page_table + (int64_t)gr.seq * p.in.max_pages) : nullptr;
      // the pool page of a step (base < hi <= kv_len: a page of the
      // sequence), wavefront-uniform; scalar loads: a vector load here would
      // make the wait for its value also wait for the direct loads in flight
      auto step_pages = [&](int s, int& pg0, int& pp0, int& pg1) {
        int lo, hi;
        const int base = step_base(s, lo, hi);
        pp0 = __builtin_amdgcn_readfirstlane(base >> sh);
        pg0 = ptab[pp0];
        pg1 = pg0;
      };
      const uint8_t* kbase = static_cast<const uint8_t*>(p.in.k) + (paged ? 0 : (int64_t)gr.key_base * KBY);
      const float* sbase = p.in.k_scale + (paged ? 0 : (int64_t)gr.key_base);
      typedef __attribute__((address_space(1))) const void gvoid;
      typedef __attribute__((address_space(3))) void lvoid;
      // direct loads of step s's rows and scales into image `img`, scales
      // `simg`; lane l's unit in instruction i is key (64 / CPK) i + l / CPK,
      // chunk (l % CPK) ^ ((l / CPK) % CPK) (the same chunk for every i)
      // The step's rows are consecutive: row(base + r) = row0 + r, so
      // instruction i reads 1 KiB at row0 * KBY + 1024 i.  Steps at a
      // range's ends clamp their keys into [lo, hi) (rows outside it are
      // never read; clamping keeps every address inside the sequence).
      auto issue_as = [&](auto paged_t, int s, uint8_t* img, float* simg, int pg0, int pp0, int pg1) {
        constexpr bool PG = decltype(paged_t)::value;
        int lo, hi;
        const int base = step_base(s, lo, hi);
        const uint32_t ln = (uint32_t)lane_fresh();
        const int rl = (int)(ln / CPK);
        const uint32_t ch = (ln % CPK) ^ ((uint32_t)rl % CPK);
        // row of the step's key 0 (wavefront-uniform)
        const int64_t row0 = PG ? ((int64_t)pg0 << sh) + (base & ((1 << sh) - 1)) : (int64_t)base;
        uint8_t* dimg = img + wave * 64 * KBY;
        if (base >= lo && base + 64 <= hi) {
          const uint8_t* src = kbase + (row0 + rl) * KBY + 16u * ch;
#pragma unroll
          for (int i = 0; i < CPK; ++i)
            __builtin_amdgcn_global_load_lds((gvoid*)(src + 1024 * i), (lvoid*)(dimg + 1024 * i), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((gvoid*)(sbase + row0 + ln), (lvoid*)(simg + wave * 64), 4, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < CPK; ++i) {
            const int r = min(max(base + (64 / CPK) * i + rl, lo), hi - 1) - base;
            const uint8_t* src = kbase + (row0 + r) * KBY + 16u * ch;
            __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)(dimg + 1024 * i), 16, 0, 0);
          }
          const int r = min(max(base + (int)ln, lo), hi - 1) - base;
          __builtin_amdgcn_global_load_lds((gvoid*)(sbase + row0 + r), (lvoid*)(simg + wave * 64), 4, 0, 0);
        }
      };
      auto issue = [&](int s, uint8_t* img, float* simg, int pg0, int pp0, int pg1) {
        if (paged) issue_as(std::true_type{}, s, img, simg, pg0, pp0, pg1);
        else issue_as(std::false_type{}, s, img, simg, pg0, pp0, pg1);
      };
      // raw fragments of blocks 2j, 2j+1 (keys r = 48 - 16 b + column) from an image
      auto read2 = [&](const uint8_t* img, const float* simg, int j, typename O::raw* rw, float* ks2) {
        const int ln = lane_fresh();
        const int c = ln & 15, g = ln >> 4;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int r = 48 - 16 * (2 * j + bb) + c;
          const uint8_t* row = img + wave * 64 * KBY + r * KBY;
          if constexpr (KBY == 128) {
            const v4i lo4 = *reinterpret_cast<const v4i*>(row + 16 * ((2 * g) ^ (r % 8)));
            const v4i hi4 = *reinterpret_cast<const v4i*>(row + 16 * ((2 * g + 1) ^ (r % 8)));
            rw[bb] = typename O::raw{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          } else {
            const v4i lo4 = *reinterpret_cast<const v4i*>(row + 16 * (g ^ (r % CPK)));
            rw[bb] = typename O::raw{lo4[0], lo4[1], lo4[2], lo4[3], 0, 0, 0, 0};
          }
          ks2[bb] = HasKScale<C>::value ? simg[wave * 64 + r] : 1.f;
        }
      };
      // candidates of step sp (scores saved in opend, key scales still in
      // that step's image)
      auto append_step = [&](int sp, const float* psimg) {
        int lo, hi;
        const int base = step_base(sp, lo, hi);
        const int ln = lane_fresh();
        const int c = ln & 15;
        int keys[4];
        bool v[4];
        float ks[4], o[4];
        const v4f o4 = opend[wave * 64 + ln];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          keys[b] = base + 48 - 16 * b + c;
          v[b] = keys[b] >= lo && keys[b] < hi;
          ks[b] = psimg[wave * 64 + 48 - 16 * b + c];
          o[b] = o4[b];
        }
        sc.template append4<true>(p, gr, region, o, ks, keys, v, shist);
      };
      // Step s from image (img, simg).  The previous step's candidates are
      // appended first and the next step's loads go out after them, into the
      // image the previous step used: the wait at the top of the following
      // step then finds both the loads and the candidate stores a whole step
      // old (loads and stores may complete in any order relative to each
      // other, so that wait covers both).
      auto do_step = [&](int s, const uint8_t* img, const float* simg, uint8_t* nimg, float* nsimg, int npg0,
                         int npp0, int npg1) {
        wait_vmem();   // this step's direct loads and the previous step's candidate stores
        if (s - kTileWaves >= wave) {
          ++nstep;
          if ((nstep & 3) == 0 || nstep == 2 || nstep == 3) sc.refresh_theta(p.topk);
          append_step(s - kTileWaves, nsimg);
        }
        if (s + kTileWaves < ns) issue(s + kTileWaves, nimg, nsimg, npg0, npp0, npg1);
        float o[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          typename O::raw rw[2];
          float ks2[2];
          read2(img, simg, j, rw, ks2);
          typename O::frag B[2][SC::STEPS];
#pragma unroll
          for (int b = 0; b < 2; ++b) O::from_raw(rw[b], B[b]);
          sc.template scoreN<2>(B, o + 2 * j);
        }
        opend[wave * 64 + lane_fresh()] = v4f{o[0], o[1], o[2], o[3]};
      };
      // page entries run two steps ahead of the scoring, the key rows one
      int pa0 = 0, qa0 = 0, pa1 = 0, pb0 = 0, qb0 = 0, pb1 = 0;
      if (wave < ns) {
        if (paged) step_pages(wave, pa0, qa0, pa1);
        issue(wave, kimg0, simg0, pa0, qa0, pa1);
      }
      if (paged && wave + kTileWaves < ns) step_pages(wave + kTileWaves, pb0, qb0, pb1);
      int last = -1;   // the last step scored, whose candidates are still to append
#pragma unroll 1
      for (int s = wave; s < ns; s += 2 * kTileWaves) {
        // even step s from image 0; step s + 8 goes to image 1
        int pc0 = 0, qc0 = 0, pc1 = 0;
        if (paged && s + 2 * kTileWaves < ns) step_pages(s + 2 * kTileWaves, pc0, qc0, pc1);
        do_step(s, kimg0, simg0, kimg1, simg1, pb0, qb0, pb1);
        last = s;
        if (s + kTileWaves >= ns) break;
        // odd step s + 8 from image 1; step s + 16 goes to image 0
        int pd0 = 0, qd0 = 0, pd1 = 0;
        if (paged && s + 3 * kTileWaves < ns) step_pages(s + 3 * kTileWaves, pd0, qd0, pd1);
        do_step(s + kTileWaves, kimg1, simg1, kimg0, simg0, pc0, qc0, pc1);
        last = s + kTileWaves;
        pb0 = pd0; qb0 = qd0; pb1 = pd1;
      }
      if (last >= 0) {
        wait_vmem();
        append_step(last, ((last - wave) / kTileWaves) % 2 == 0 ? simg0 : simg1);
      }
      sc.close(p, gr, region, shist);
      sc.finish(p, region);
      return;
    }
    if (!it.gather) {
      // range walk with the next step's key bytes in flight while the current
      // step is scored (half steps of two 16-key blocks, as the list kernel)
      const int na = it.a1 > it.a0 ? (it.a1 - it.a0 + 63) / 64 : 0;
      const int ns = na + (it.b1 > it.b0 ? (it.b1 - it.b0 + 63) / 64 : 0);
      auto step_kb = [&](int s, int& lo, int& hi) -> int {
        const bool ra = s < na;
        lo = ra ? it.a0 : it.b0;
        hi = ra ? it.a1 : it.b1;
        return hi - 16 - 64 * (ra ? s : s - na);
      };
      typename O::raw rn[2];
      float ksn[2];
      auto fetch = [&](int h) {
        int lo, hi;
        const int kb = step_kb(h >> 1, lo, hi) - 32 * (h & 1);
        const int cl = sc.col();
        int64_t row[2];
        bool ok[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int key = kb - 16 * b + cl;
          ok[b] = key >= lo && key < hi;
          row[b] = ok[b] ? key_row(p.in, gr.key_base, gr.seq, key) : 0;
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          ksn[b] = 1.f;
          if (ok[b]) {
            O::load_raw(kbytes + row[b] * SC::KBYTES, sc.g(), rn[b]);
            if constexpr (HasKScale<C>::value) ksn[b] = p.in.k_scale[row[b]];
          } else {
            rn[b] = typename O::raw{};
          }
        }
      };
      if (wave < ns) fetch(2 * wave);
#pragma unroll 1
      for (int s = wave; s < ns; s += kTileWaves) {
        int lo, hi;
        const int kb = step_kb(s, lo, hi);
        int keys[4];
        bool v[4];
        float ks[4], o[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          keys[b] = kb - 16 * b + sc.col();
          v[b] = keys[b] >= lo && keys[b] < hi;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          typename O::frag B[2][SC::STEPS];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            O::from_raw(rn[b], B[b]);
            ks[2 * j + b] = ksn[b];
          }
          if (j == 0) fetch(2 * s + 1);
          else if (s + kTileWaves < ns) fetch(2 * (s + kTileWaves));
          sc.template scoreN<2>(B, o + 2 * j);
        }
        sc.template append4<true>(p, gr, region, o, ks, keys, v, shist);
        after_step();
      }
      sc.close(p, gr, region, shist);
      sc.finish(p, region);
      return;
    }
  }
  if (!it.gather) {
    const int na = it.a1 > it.a0 ? (it.a1 - it.a0 + 63) / 64 : 0;
    const int ns = na + (it.b1 > it.b0 ? (it.b1 - it.b0 + 63) / 64 : 0);
#pragma unroll 1
    for (int s = wave; s < ns; s += kTileWaves) {
      const bool ra = s < na;
      const int lo = ra ? it.a0 : it.b0, hi = ra ? it.a1 : it.b1;
      const int kb = hi - 16 - 64 * (ra ? s : s - na);
      int keys[4];
      bool v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        keys[b] = kb - 16 * b + sc.col();
        v[b] = keys[b] >= lo && keys[b] < hi;
      }
      step4(keys, v);
    }
  } else {
    // share a0 of a1 of the group's survivor list, 64 entries per step
    const int32_t* lst = p.list_stride > 0 ? p.lists + (int64_t)it.group * p.list_stride
                                           : p.lists + gr.list_off + (p.list_start != nullptr ? p.list_start[it.group] : 0);
    const int len = p.list_len[it.group];
    const int e0 = (int)(((int64_t)len * it.a0 / it.a1) & ~15LL);
    const int e1 = (it.a0 == it.a1 - 1) ? len : (int)(((int64_t)len * (it.a0 + 1) / it.a1) & ~15LL);
#pragma unroll 1
    for (int e = e0 + 64 * wave; e < e1; e += 64 * kTileWaves) {
      int keys[4];
      bool v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i0 = e + 16 * b + sc.col();
        v[b] = i0 < e1;
        keys[b] = v[b] ? lst[i0] : 0;
      }
      step4(keys, v);
    }
  }
  sc.close(p, gr, region, shist);
  sc.finish(p, region);
}

// ---------------------------------------------------------------------------
// 8 wavefronts (consecutive query groups of one sequence) share LDS key tiles.
// Range mode: [a0,a1) then [b0,b1), each from the top tile down.  Gather mode
// (survivor pass only): share a0 of a1 of the tile's union survivor list,
// from its last entry down; every listed key lies before the tile's first
// query, so it is visible to all of them.  PAGED: keys go through the page
// table; otherwise a key row is addressed from a single base.
// ---------------------------------------------------------------------------
template <int C, int H, int D, int ROLE, bool PAGED>
__global__ __launch_bounds__(64 * kTileWaves) void score_tiled_kernel(const ScoreLaunch p) {
  using SC = Scorer<C, H, D>;
  using O = typename SC::O;
  constexpr int KB = SC::KBYTES;
  constexpr int ROW = KB + 16;                       // padded LDS row: conflict-free 16-byte reads
  constexpr int CPK = KB / 16;                       // 16-byte chunks per key
  constexpr int TK = kTileKeys;                      // keys per LDS tile (one 64-key scoring step)
  constexpr int NCH = (TK * CPK + 64 * kTileWaves - 1) / (64 * kTileWaves);
  // 16-key blocks per scoring step: as many as the key fragments' registers allow
  constexpr int FB = (int)sizeof(typename O::frag) * SC::STEPS;   // bytes of one block's key fragment per lane
  constexpr int NBK = FB <= 32 ? 4 : (FB <= 64 ? 2 : 1);
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][TK * ROW];
  __shared__ float kscale[2][TK];
  __shared__ int32_t kid[2][TK];                     // gather mode: the tile's key positions (-1: none)
  __shared__ __attribute__((aligned(16))) float wl[kTileWaves][SC::QW * (H + SC::S)];
  __shared__ uint32_t hist[kTileWaves][256];
  __shared__ uint32_t qhist[kTileWaves][SC::QW * kHistBins];

  if (skip_launch(p.mode, p.run_if)) return;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x) >> 6;   // wavefront-uniform
  const WorkItem it = p.items[p.order != nullptr ? p.order[blockIdx.x] : (int)blockIdx.x];
  const int ngroups = it.pad;                        // query groups in this tile
  if (p.flag_mode == 1) {
    bool all = true;
    for (int i = 0; i < ngroups; ++i) all = all && (p.tile_flags[it.group + i] != 0);
    if (!all) return;  // the list kernel scores this tile's survivors
  }
  const bool active = wave < ngroups;
  const GroupInfo gr = p.groups[it.group + (active ? wave : 0)];
  const GroupInfo g0 = p.groups[it.group];
  // gather mode: entries [e0, e1) of the union list; a short list is cut into
  // fewer shares of at least kUnionMinShare keys, and the items of the unused
  // shares leave here
  constexpr bool kGatherRole = (ROLE == ROLE_SURVIVORS);
  const bool gather = kGatherRole && it.gather != 0;
  const int32_t* ulist = p.lists + g0.list_off;
  int e0 = 0, e1 = 0;
  if (gather) {
    const int len = p.list_len[it.group];
    const int nsh = min(it.a1, max(1, (len + kUnionMinShare - 1) / kUnionMinShare));
    if (it.a0 >= nsh) return;
    e0 = (int)((int64_t)len * it.a0 / nsh);
    e1 = (int)((int64_t)len * (it.a0 + 1) / nsh);
  }
  SC sc;
  sc.init(p, gr, it.region, wl[wave], qhist[wave], active);
  sc.set_part(p, it);

  const int na = gather ? 0 : ((it.a1 > it.a0) ? (it.a1 - it.a0 + TK - 1) / TK : 0);
  const int nbt = gather ? (e1 - e0 + TK - 1) / TK : ((it.b1 > it.b0) ? (it.b1 - it.b0 + TK - 1) / TK : 0);
  const int ntiles = na + nbt;
  // contiguous storage: row r of the sequence's keys at kseq + r * KB
  const uint8_t* kseq = static_cast<const uint8_t*>(p.in.k) + (PAGED ? 0 : (int64_t)g0.key_base * KB);
  const float* sseq = p.in.k_scale + (PAGED ? 0 : (int64_t)g0.key_base);
  const int last0 = gr.pos0;                         // every query of the group sees keys <= last0

  v4i stage[NCH];
  float stage_s = 1.f;
  int stage_id = -1;
  // Gather mode: the list entries (key positions) of a tile are loaded one
  // tile ahead of its key rows, so a tile's rows wait for one memory latency,
  // not for the list read and then the rows.  The last iteration's reload
  // stages an empty tile into the idle buffer; nothing reads it.
  int idn[NCH];
  int idn_s = -1;
  auto load_ids = [&](int tt) {
    const int tid = lane_fresh() + 64 * wave;
    const int ib = e1 - TK * (tt + 1);               // list index of tile tt's slot 0
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int slot = (tid + c * 64 * kTileWaves) / CPK;
      const int idx = ib + slot;
      idn[c] = (tt < ntiles && slot < TK && idx >= e0) ? ulist[idx] : -1;
    }
    if (tid < TK) {
      const int idx = ib + tid;
      idn_s = (tt < ntiles && idx >= e0) ? ulist[idx] : -1;
    }
  };
  auto fetch_gather = [&](int t) {
    const int tid = lane_fresh() + 64 * wave;
    int idc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) idc[c] = idn[c];
    const int ids = idn_s;
    load_ids(t + 1);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int part = (tid + c * 64 * kTileWaves) % CPK;
      if (idc[c] >= 0) {
        const int64_t row = PAGED ? key_row(p.in, g0.key_base, g0.seq, idc[c]) : (int64_t)idc[c];
        stage[c] = *reinterpret_cast<const v4i*>(kseq + row * KB + part * 16);
      } else {
        stage[c] = v4i{0, 0, 0, 0};
      }
    }
    if (tid < TK) {
      stage_id = ids;
      if constexpr (HasKScale<C>::value) {
        if (ids >= 0)
          stage_s = PAGED ? p.in.k_scale[key_row(p.in, g0.key_base, g0.seq, ids)] : sseq[(uint32_t)ids];
        else
          stage_s = 0.f;
      }
    }
  };
  auto fetch = [&](int t) {
    if (kGatherRole && gather) {
      fetch_gather(t);
      return;
    }
    const bool ra = t < na;
    const int lo = ra ? it.a0 : it.b0, hi = ra ? it.a1 : it.b1;
    const int kb = hi - TK * ((ra ? t : t - na) + 1);
    if (!PAGED && kb >= lo && kb + TK <= hi) {
      // every key of the tile in range: its rows are TK * KB contiguous bytes
      // from a wavefront-uniform base, chunk ch at byte 16 ch
      const int tid = lane_fresh() + 64 * wave;
      const uint8_t* kt = kseq + (uint32_t)kb * (uint32_t)KB;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int ch = tid + c * 64 * kTileWaves;
        if ((TK * CPK) % (64 * kTileWaves) == 0 || ch < TK * CPK)
          stage[c] = *reinterpret_cast<const v4i*>(kt + (uint32_t)ch * 16u);
      }
      if constexpr (HasKScale<C>::value) {
        if (tid < TK) stage_s = sseq[(uint32_t)kb + (uint32_t)tid];
      }
      return;
    }
    const int tid = lane_fresh() + 64 * wave;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * 64 * kTileWaves;
      const int slot = ch / CPK, part = ch % CPK;
      const int key = kb + slot;
      if (slot < TK && key >= lo && key < hi) {
        if constexpr (PAGED) {
          const int64_t row = key_row(p.in, g0.key_base, g0.seq, key);
          stage[c] = *reinterpret_cast<const v4i*>(kseq + row * KB + part * 16);
        } else {
          stage[c] = *reinterpret_cast<const v4i*>(kseq + ((uint32_t)key * (uint32_t)KB + (uint32_t)(part * 16)));
        }
      } else {
        stage[c] = v4i{0, 0, 0, 0};
      }
    }
    if constexpr (HasKScale<C>::value) {
      if (tid < TK) {
        const int key = kb + tid;
        if (key >= lo && key < hi)
          stage_s = PAGED ? p.in.k_scale[key_row(p.in, g0.key_base, g0.seq, key)] : sseq[(uint32_t)key];
        else
          stage_s = 0.f;
      }
    }
  };
  auto commit = [&](int bufi) {
    const int tid = lane_fresh() + 64 * wave;
    wait_vmem();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      // chunk ch = (slot, part) goes to slot * ROW + 16 part = 16 (ch + slot)
      const int ch = tid + c * 64 * kTileWaves;
      const int slot = ch / CPK;
      if (slot < TK) *reinterpret_cast<v4i*>(&ktile[bufi][16 * (ch + slot)]) = stage[c];
    }
    if (tid < TK) {
      kscale[bufi][tid] = stage_s;
      if (kGatherRole) kid[bufi][tid] = stage_id;
    }
  };

  drain_memory();   // the query fragments of init, before the prefetching loop
  // Tile t+1 is loaded while tile t is scored and is written to LDS before
  // tile t's candidates are appended, so the wait for the loads never
  // includes candidate stores just issued (one counter covers both).  The
  // last iteration reloads its own tile into the idle buffer: an unconditional
  // load and wait leave nothing pending into the next iteration on any path.
  if (ntiles > 0) {
    if (kGatherRole && gather) load_ids(0);
    fetch(0);
    commit(0);
  }
  __syncthreads();
  auto range_epilogue = [&](const float* o4, const float* ks4, int kh, int lo, int hi) {
    // whole step inside the range and visible to every query of the group
    const bool full = kh >= lo && kh + kTileKeys <= hi && kh + kTileKeys - 1 <= last0;
    if (full) {
      // key positions kh + 16 b + column, formed only for taken scores
      sc.template append4<false, true>(p, gr, it.region, o4, ks4, nullptr, nullptr, hist[wave], kh);
    } else {
      const int cl = sc.col();
      int keys[4];
      bool kv[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        keys[b] = kh + b * 16 + cl;
        kv[b] = keys[b] >= lo && keys[b] < hi;
      }
      sc.template append4<true>(p, gr, it.region, o4, ks4, keys, kv, hist[wave]);
    }
  };
#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    const int bufi = t & 1;
    fetch(min(t + 1, ntiles - 1));
    const bool ra = t < na;
    const int lo = ra ? it.a0 : it.b0, hi = ra ? it.a1 : it.b1;
    const int kb = hi - TK * ((ra ? t : t - na) + 1);
    float o[4];
    if (active) {
      // one fresh lane id for every fragment address of the tile: the blocks'
      // LDS reads then differ by immediate offsets only
      const int ln = lane_fresh();
      const int fcol = ln & 15, fg = ln >> 4;
#pragma unroll
      for (int hb = 0; hb < 4 / NBK; ++hb) {
        typename O::frag B[NBK][SC::STEPS];
#pragma unroll
        for (int b = 0; b < NBK; ++b) O::load_k(&ktile[bufi][((NBK * hb + b) * 16 + fcol) * ROW], fg, B[b]);
        // all blocks' fragments in flight together: one LDS wait, not one per block
#pragma unroll
        for (int b = 0; b < NBK; ++b)
#pragma unroll
          for (int s = 0; s < SC::STEPS; ++s) asm volatile("" : "+v"(B[b][s]));
        sc.template scoreN<NBK>(B, o + NBK * hb);
      }
    }
    commit(bufi ^ 1);
    if (active) {
      const int cl = sc.col();
      float ks[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) ks[b] = HasKScale<C>::value ? kscale[bufi][b * 16 + cl] : 1.f;
      if (kGatherRole && gather) {
        int keys[4];
        bool kv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          keys[b] = kid[bufi][b * 16 + cl];
          kv[b] = keys[b] >= 0;
        }
        // every slot of the tile filled: each listed key lies before the
        // tile's first query
        if (e1 - TK * (t + 1) >= e0)
          sc.template append4<false>(p, gr, it.region, o, ks, keys, kv, hist[wave]);
        else
          sc.template append4<true>(p, gr, it.region, o, ks, keys, kv, hist[wave]);
      } else {
        range_epilogue(o, ks, kb, lo, hi);
      }
      if ((t & (kRefreshTiles - 1)) == kRefreshTiles - 1 && sc.dirty) sc.refresh_theta(p.topk);
    }
    __syncthreads();
  }
  if (active) {
    sc.close(p, gr, it.region, hist[wave]);
    sc.finish(p, it.region);
  }
}

// ---------------------------------------------------------------------------
// launcher for one operand combination (instantiated per score_<combo>.hip)
// ---------------------------------------------------------------------------
template <int C, int H, int D, int ROLE>
static hipError_t launch_score_r(const ScoreLaunch& p, hipStream_t s) {
  if (p.tiled == 2)
    hipLaunchKernelGGL((score_split_kernel<C, H, D, ROLE>), dim3(p.n_items), dim3(64 * kTileWaves), 0, s, p);
  else if (p.tiled && p.in.page_table != nullptr)
    hipLaunchKernelGGL((score_tiled_kernel<C, H, D, ROLE, true>), dim3(p.n_items), dim3(64 * kTileWaves), 0, s, p);
  else if (p.tiled)
    hipLaunchKernelGGL((score_tiled_kernel<C, H, D, ROLE, false>), dim3(p.n_items), dim3(64 * kTileWaves), 0, s, p);
  else
    hipLaunchKernelGGL((score_list_kernel<C, H, D, ROLE>), dim3(p.n_items), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int C, int H, int D>
static hipError_t launch_score_t(const ScoreLaunch& p, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  switch (p.role) {
    case ROLE_SEED: return launch_score_r<C, H, D, ROLE_SEED>(p, s);
    case ROLE_SURVIVORS: return launch_score_r<C, H, D, ROLE_SURVIVORS>(p, s);
    default: return launch_score_r<C, H, D, ROLE_DENSE>(p, s);
  }
}

template <int C>
static hipError_t launch_score_c(int H, int d, const ScoreLaunch& p, hipStream_t s) {
#define DOSA_HD(HH, DD) \
  if (HP == HH && d == DD) return launch_score_t<C, HH, DD>(p, s);
  const int HP = padded_heads(H);
  DOSA_HD(8, 64) DOSA_HD(16, 64) DOSA_HD(32, 64) DOSA_HD(64, 64)
  DOSA_HD(8, 128) DOSA_HD(16, 128) DOSA_HD(32, 128) DOSA_HD(64, 128)
#undef DOSA_HD
  return hipErrorInvalidValue;
}

}  // namespace dosa

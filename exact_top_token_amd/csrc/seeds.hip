// Extra seed keys supplied by the caller (the DoSA transcript, Experiments:
// decode reuses the scores of recently selected keys; the PIVOT record: one
// candidate set per group of nearby queries).  They only raise the seed
// threshold tau: every extra key is scored exactly with all heads into
// candidate regions that the threshold select reads and the final merge does
// not, so a key listed here and also kept by the certificate is counted once.
//
// A query group scores the union of its queries' rows (every score of a
// visible key, exact and distinct from the others, is a valid candidate for
// the K-th largest, whichever query listed it).  The union is restricted to
// the group's bounded keys: the seed prefix and window are scored already,
// and the bounded range lies before the group's first query, so every listed
// key is visible to all of its queries.
#include <climits>

#include "dosa_device.h"
#include "dosa_internal.h"

namespace dosa {
namespace {

constexpr int kUnionThreads = 1024;

// One workgroup per query group: gather the rows, drop keys outside the
// bounded range, bitonic sort in LDS (ascending, INT_MAX as filler), keep the
// first key of every run of equal keys, write the list in order.
__global__ __launch_bounds__(kUnionThreads) void seed_union_kernel(const SeedUnionLaunch p) {
  __shared__ int32_t v[kSeedUnionMax];
  __shared__ uint32_t wcount[kUnionThreads / 64];
  if (skip_launch(p.mode, p.run_if)) return;
  const GroupInfo g = p.groups[blockIdx.x];
  const int n = g.nq * p.seed_count;
  int m = 1;
  while (m < n) m <<= 1;
  const int lo = g.bound_lo, hi = g.bound_lo + max(g.n_bounded, 0);
  const int32_t* src = p.seed_idx + (int64_t)g.q_row0 * p.seed_count;
  for (int i = threadIdx.x; i < m; i += kUnionThreads) {
    int x = INT_MAX;
    if (i < n) {
      const int y = src[i];
      if (y >= lo && y < hi) x = y;
    }
    v[i] = x;
  }
  __syncthreads();
  for (int k = 2; k <= m; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += kUnionThreads) {
        const int l = i ^ j;
        if (l > i) {
          const int a = v[i], b = v[l];
          if ((a > b) == ((i & k) == 0)) {
            v[i] = b;
            v[l] = a;
          }
        }
      }
      __syncthreads();
    }
  int32_t* out = p.lists + (int64_t)blockIdx.x * p.stride;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  uint32_t base = 0;
  for (int c = 0; c < m; c += kUnionThreads) {
    const int i = c + (int)threadIdx.x;
    const int x = i < m ? v[i] : INT_MAX;
    const bool keep = x != INT_MAX && (i == 0 || v[i - 1] != x);
    const unsigned long long bal = __ballot(keep);
    if (lane == 0) wcount[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = base, total = base;
    for (int w = 0; w < kUnionThreads / 64; ++w) {
      if (w < wave) before += wcount[w];
      total += wcount[w];
    }
    if (keep) out[before + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull))] = x;
    base = total;
    __syncthreads();
  }
  if (threadIdx.x == 0) p.list_len[blockIdx.x] = (int32_t)base;
}

}  // namespace

hipError_t launch_seed_union(const SeedUnionLaunch& p, hipStream_t s) {
  if (p.n_groups == 0 || p.seed_count <= 0) return hipSuccess;
  hipLaunchKernelGGL(seed_union_kernel, dim3(p.n_groups), dim3(kUnionThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dosa

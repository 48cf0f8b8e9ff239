// C-ABI entry points: argument checks, work planning, workspace layout and
// kernel launches on the caller's stream.  No allocation, no host sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dosa_device.h"
#include "dosa_internal.h"

using namespace dosa;

namespace {

thread_local std::string g_err;

// ---------------------------------------------------------------------------
// optional per-pass event timing
// ---------------------------------------------------------------------------
enum PassId { P_NORMS = 0, P_SCORE_SEED, P_SELECT_SEED, P_PLAN, P_BOUND, P_COMPACT, P_SURV_TILES, P_SURV_LISTS,
              P_SCORE_DENSE, P_SELECT_FINAL, P_PREP, P_PROBE, P_SEED_EXTRA, P_COUNT };
const char* const kPassNames[P_COUNT] = {"key_norms", "score_seed", "select_seed", "plan", "bound", "compact",
                                         "score_survivor_tiles", "score_survivor_lists", "score_dense",
                                         "select_final", "prep", "probe", "seed_extra"};

struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, size_t>> recs;   // (pass, index of start event; stop = +1)
  hipEvent_t next() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
thread_local Profiler g_prof;

struct PassScope {
  hipStream_t s;
  hipEvent_t stop = nullptr;
  PassScope(int pass, hipStream_t st) : s(st) {
    if (!g_prof.on) return;
    const size_t at = g_prof.used;
    hipEvent_t a = g_prof.next(), b = g_prof.next();
    if (!a || !b) return;
    hipEventRecord(a, s);
    stop = b;
    g_prof.recs.push_back({pass, at});
  }
  ~PassScope() {
    if (stop) hipEventRecord(stop, s);
  }
};

int fail_hip(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return DOSA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The certificate stages of a call with a probe run on a side stream of the
// library's own, next to the dense alternative on the caller's stream: the
// probe's decision lets exactly one of the two do work, and the other's
// launches return at once without delaying it.  One side stream per device,
// created on first use (default priority) and kept until the process ends.
// Each call forks it from the caller's stream after the probe and joins it
// back before the final selection, with events of its own, so the caller's
// stream order covers all of the call's work (graph capture included).  Calls
// that run at the same time on one device share the side stream: their
// certificate stages then run one after the other.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
constexpr int kSideStreamMaxItems = 512;   // dense work items of a call that still takes the side stream
constexpr uint64_t kSideStreamMinPairs = uint64_t(1) << 26;   // causal pairs of a call that takes the side stream
std::once_flag g_side_once[kMaxDevices];
hipStream_t g_side[kMaxDevices] = {};
hipError_t g_side_err[kMaxDevices] = {};

hipError_t side_stream(hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_side_once[dev], [dev]() { g_side_err[dev] = hipStreamCreateWithFlags(&g_side[dev], hipStreamNonBlocking); });
  if (g_side_err[dev] != hipSuccess) return g_side_err[dev];
  *out = g_side[dev];
  return hipSuccess;
}

// Fork of the side stream from the caller's stream; the destructor joins it
// back (also on an early error return), so nothing of the call is left
// unordered with the caller's later work.
struct SideFork {
  hipStream_t main = nullptr, side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipError_t open(hipStream_t caller) {
    main = caller;
    // per-pass event timing keeps every pass on the caller's stream, so each
    // pass's span is its own launch (not the wait for CUs held by the other)
    if (g_prof.on) return hipSuccess;
    hipError_t e = side_stream(&side);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(fork, main);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, fork, 0);
    if (e != hipSuccess) side = nullptr;   // stay on the caller's stream
    return e;
  }
  hipError_t close() {
    hipError_t e = hipSuccess;
    if (side != nullptr) {
      e = hipEventRecord(join, side);
      if (e == hipSuccess) e = hipStreamWaitEvent(main, join, 0);
      side = nullptr;
    }
    if (fork) hipEventDestroy(fork);
    if (join) hipEventDestroy(join);
    fork = join = nullptr;
    return e;
  }
  ~SideFork() { close(); }
};

int combo_of(int qd, int kd) {
  if (qd == DOSA_F32 && kd == DOSA_F32) return C_F32;
  if (qd == DOSA_BF16 && kd == DOSA_BF16) return C_BF16;
  if (qd == DOSA_FP8_E4M3FN && kd == DOSA_FP8_E4M3FN) return C_FP8;
  if (qd == DOSA_BF16 && kd == DOSA_FP8_E4M3FN) return C_BF16Q_FP8K;
  return -1;
}

int qbytes(int qd) { return qd == DOSA_F32 ? 4 : (qd == DOSA_BF16 ? 2 : 1); }

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Everything the planner derives from the shapes.
struct Plan {
  int combo = -1, QW = 4, J = 1, R = 1, cap = 0, F = 0, W = 0;
  bool dense = true;
  int64_t total_q = 0, total_k = 0;
  std::vector<GroupInfo> groups;
  std::vector<WorkItem> items;       // dense: scoring items; DoSA: seed, tiled-survivor, list-survivor items
  std::vector<WorkItem> seed_items, surv_tiled_items, surv_list_items, bound_items, dense_items,
      x_items;                       // DoSA with extra seed keys: their scoring items (regions Js..Js+X-1)
  // DoSA in two rounds (DOSA_TWO_ROUNDS, calls with query tiles): each round's
  // groups (bounded range: round 1 the newer half, round 2 the older half),
  // round 2's bound items and survivor items (regions Js+X+J..Js+X+2J-1)
  bool two_rounds = false;
  std::vector<GroupInfo> groups_r1, groups_r2;
  std::vector<WorkItem> bound_items2, surv_tiled_items2, surv_list_items2;
  size_t o_groups1 = 0, o_groups2 = 0;
  bool probe = false;                // DoSA: plan the last tile first, score densely if it cannot prune
  int probe_group = 0, probe_ngroups = 0, probe_q0 = 0, probe_nq = 0, Jd = 0;
  int bound_gpw = 1;                 // query groups per wavefront of the tiled bound kernel
  bool tiled = true;
  int RW = 1;                        // candidate regions per item region: 1, or kTileWaves for the split
                                     // kernel (decode-like batches: one region per wavefront)
  int bound_splits = 1;
  int Js = 1;                        // DoSA: regions of the seed pass
  int X = 0;                         // DoSA: regions of the extra seed keys (after the seed regions)
  int n_parts = 0;                   // split-threshold slots per query (tiled dense / seed launches)
  int64_t x_stride = 0;              // entries per group of the extra seed lists
  int n_tiles = 0;                   // query tiles (seed items 0 .. n_tiles*Js-1 are Js per tile, tile order)
  int mask_words = 0;
  int64_t list_total = 0;
  int64_t n_blocks = 0;              // 64-key blocks of all sequences (key-block summaries)
  // workspace offsets
  size_t o_groups = 0, o_items = 0, o_cand = 0, o_counts = 0, o_tau = 0, o_rows = 0, o_coef = 0,
         o_norms = 0, o_masks = 0, o_lists = 0, o_listlen = 0, o_seqinfo = 0, o_gflags = 0, o_flag = 0,
         o_lrows = 0, o_lsig = 0, o_lerr = 0, o_mode = 0, o_tshare = 0, o_order = 0, o_blk_code = 0, o_blk_info = 0,
         o_liststart = 0, o_xlists = 0, o_xlen = 0, o_tpart = 0, total = 0;
  uint64_t pairs_total = 0;
};

int check_shapes(int32_t batch, const int32_t* q_lens, const int32_t* kv_lens, int32_t H, int32_t d,
                 int32_t topk, int32_t q_dtype, int32_t k_dtype) {
  if (batch < 0 || (batch > 0 && (q_lens == nullptr || kv_lens == nullptr))) {
    g_err = "batch < 0 or q_lens/kv_lens NULL";
    return DOSA_ERR_INVALID_ARG;
  }
  if (H <= 0 || d <= 0 || topk <= 0) {
    g_err = "H, d and topk must be positive";
    return DOSA_ERR_INVALID_ARG;
  }
  for (int b = 0; b < batch; ++b) {
    if (q_lens[b] < 0 || kv_lens[b] < 0 || q_lens[b] > kv_lens[b]) {
      g_err = "sequence " + std::to_string(b) + ": need 0 <= q_len <= kv_len";
      return DOSA_ERR_INVALID_ARG;
    }
  }
  const int combo = combo_of(q_dtype, k_dtype);
  if (combo < 0 || !combo_supported(combo, H, d) || topk > 4096) {
    g_err = "unsupported dtype combination, H, d or topk";
    return DOSA_ERR_UNSUPPORTED;
  }
  // Index arithmetic limits: query rows, key rows and per-key norm slots are
  // int32; a contiguous sequence's key rows are addressed by 32-bit byte
  // offsets from its first row.
  int64_t tq = 0, tk = 0, kmax = 0;
  for (int b = 0; b < batch; ++b) {
    tq += q_lens[b];
    tk += kv_lens[b];
    kmax = std::max<int64_t>(kmax, kv_lens[b]);
  }
  const int64_t kbytes = (k_dtype == DOSA_F32) ? 4 : (k_dtype == DOSA_BF16 ? 2 : 1);
  if (tq >= (int64_t(1) << 31) || tk >= (int64_t(1) << 31) || kmax * d * kbytes >= (int64_t(1) << 32)) {
    g_err = "too many queries or keys for 32-bit row indices";
    return DOSA_ERR_UNSUPPORTED;
  }
  return DOSA_OK;
}

int resolve_cfg(const dosa_config* in, int32_t topk, dosa_config* out) {
  dosa_default_config(topk, out);
  if (in) {
    *out = *in;
    if (out->num_proxies < 0 || out->num_proxies > 3 || out->seed_window < 0 || out->seed_prefix < 0 ||
        out->key_splits < 0 || !(out->neg_support_frac >= 0.f && out->neg_support_frac <= 1.f)) {
      g_err = "config out of range";
      return DOSA_ERR_INVALID_ARG;
    }
    if (out->buffer_cap != 0 && out->buffer_cap < topk + 64) {
      g_err = "buffer_cap must be >= topk + 64";
      return DOSA_ERR_INVALID_ARG;
    }
    if (out->seed_count < 0 || out->seed_count > kMaxSeedCount || (out->seed_count > 0 && out->seed_idx == nullptr)) {
      g_err = "seed_count must be in 0.." + std::to_string(kMaxSeedCount) + ", with seed_idx when positive";
      return DOSA_ERR_INVALID_ARG;
    }
    if (out->seed_idx == nullptr) out->seed_count = 0;
  }
  return DOSA_OK;
}

struct TileInfo {
  int first, n, n_last, seq;
};

// Work items of one launch, longest key range first: the dispatcher hands out
// workgroups in item order, so the short items fill the tail of the launch
// (longest-processing-time-first scheduling).  Stable, so the order of equal
// items stays the plan's.
void longest_first(std::vector<WorkItem>& v, size_t from) {
  std::stable_sort(v.begin() + (std::ptrdiff_t)from, v.end(), [](const WorkItem& x, const WorkItem& y) {
    return (x.a1 - x.a0) + (x.b1 - x.b0) > (y.a1 - y.a0) + (y.b1 - y.b0);
  });
}

// Key splits of one query share their running thresholds (see ScoreLaunch).
constexpr bool kShareTheta = true;

// Items per call of the split kernel (decode-like batches): one 8-wavefront
// workgroup per CU.
constexpr int64_t kSplitItems = 256;

// Groups planned by the probe of a call without query tiles.
constexpr int kProbeGroups = 256;

// Split choice: enough work items to fill the GPU (target items), keeping at
// least min_keys keys per split.
int choose_splits(int64_t n_units, int64_t avg_keys, int64_t target, int64_t min_keys) {
  int J = 1;
  while (n_units * J < target && avg_keys / (2 * J) >= min_keys && J < 64) J *= 2;
  return J;
}

void build_plan(Plan& P, int32_t batch, const int32_t* q_lens, const int32_t* kv_lens, int32_t H, int32_t d,
                int32_t topk, int32_t q_dtype, int32_t k_dtype, bool paged, bool dense,
                const dosa_config& cfg) {
  P.combo = combo_of(q_dtype, k_dtype);
  P.QW = queries_per_wave(P.combo, padded_heads(H), d);
  P.dense = dense;
  P.F = cfg.seed_prefix;
  P.W = std::max(cfg.seed_window, 64);
  const int TW = tile_waves();
  int64_t cq = 0, ck = 0, cb = 0;
  uint64_t pairs = 0;
  std::vector<TileInfo> tiles;
  for (int b = 0; b < batch; ++b) {
    const int m = q_lens[b], n = kv_lens[b];
    for (int i = 0; i < m; i += P.QW) {
      GroupInfo g{};
      g.seq = b;
      g.q_row0 = (int32_t)(cq + i);
      g.nq = std::min(P.QW, m - i);
      g.pos0 = n - m + i;
      g.key_base = paged ? 0 : (int32_t)ck;
      g.norm_base = (int32_t)ck;
      g.blk_base = (int32_t)cb;
      const int gi = (int)P.groups.size();
      if (tiles.empty() || tiles.back().seq != b || tiles.back().n == TW) tiles.push_back({gi, 0, 0, b});
      tiles.back().n += 1;
      tiles.back().n_last = g.pos0 + g.nq;
      P.groups.push_back(g);
    }
    pairs += (uint64_t)m * (uint64_t)(n - m + 1) + (uint64_t)m * (uint64_t)(m - 1) / 2;
    cq += m;
    ck += n;
    cb += (n + kKeyBlock - 1) / kKeyBlock;
  }
  P.n_blocks = cb;
  for (auto& t : tiles)
    for (int i = 0; i < t.n; ++i) {
      P.groups[t.first + i].tile_first = t.first;
      P.groups[t.first + i].tile_n = t.n;
    }
  P.total_q = cq;
  P.total_k = ck;
  P.n_tiles = (int)tiles.size();
  P.pairs_total = pairs;
  const int G = (int)P.groups.size();
  const int NT = (int)tiles.size();
  int64_t key_sum = 0;
  for (auto& t : tiles) key_sum += t.n_last;
  const int64_t avg_keys = NT ? key_sum / NT : 0;
  // Tiles that hold few groups waste the tiled kernel's wavefronts: decode-
  // like batches are scored by the split kernel instead (a workgroup's 8
  // wavefronts on one group's keys), in items of balanced key counts.
  P.tiled = (NT > 0) && (2 * G >= TW * NT);
  P.RW = P.tiled ? 1 : TW;
  // balanced items of the split kernel: key ranges of at most `chunk` keys,
  // the smallest chunk (a multiple of 64, at least 1024) for which the ranges
  // of all groups make at most kSplitItems items -- one 8-wavefront workgroup
  // per CU, all in one round, so no CU runs a second item while the others idle
  auto split_chunk = [&](const std::vector<int64_t>& lens) -> int64_t {
    int64_t lo = 1024, hi = 1024;
    for (int64_t n : lens) hi = std::max(hi, (n + 63) / 64 * 64);
    auto items = [&](int64_t c) {
      int64_t k = 0;
      for (int64_t n : lens) k += (n + c - 1) / c;
      return k;
    };
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2 / 64 * 64;
      if (mid <= lo) break;
      if (items(mid) <= kSplitItems) hi = mid;
      else lo = mid + 64;
    }
    return items(lo) <= kSplitItems ? lo : hi;
  };
  auto split_range = [&](int gi, int lo_all, int hi_all, int region0, int64_t chunk, std::vector<WorkItem>& out) {
    const int n = hi_all - lo_all;
    const int J = cfg.key_splits > 0 ? cfg.key_splits : (int)std::max<int64_t>(1, (n + chunk - 1) / chunk);
    for (int r = 0; r < J; ++r) {
      const int64_t len = n;
      const int lo = lo_all + (int)((len * r / J) / 64 * 64);
      const int hi = (r == J - 1) ? hi_all : lo_all + (int)((len * (r + 1) / J) / 64 * 64);
      WorkItem it{};
      it.group = gi;
      it.region = region0 + r;
      it.nparts = J;
      if (lo == 0) {
        it.a0 = 0; it.a1 = std::min(64, hi);   // the attention-sink keys first, then newest to oldest
        it.b0 = it.a1; it.b1 = hi;
      } else {
        it.a0 = it.a1 = lo;
        it.b0 = lo; it.b1 = hi;
      }
      out.push_back(it);
    }
    return J;
  };
  // work items that give every SIMD two wavefronts of tiled scoring
  const int64_t tiled_target = 2048 / TW;
  auto range_split = [](int lo_all, int hi_all, int r, int J, int align, int& lo, int& hi) {
    const int64_t len = hi_all - lo_all;
    lo = lo_all + (int)((len * r / J) / align * align);
    hi = (r == J - 1) ? hi_all : lo_all + (int)((len * (r + 1) / J) / align * align);
  };
  // dense scoring of whole tiles: J key ranges per tile, regions 0..J-1
  auto dense_tiled_items = [&](std::vector<WorkItem>& out) {
    const int J = cfg.key_splits > 0 ? cfg.key_splits : choose_splits(NT, avg_keys, tiled_target, 1024);
    const size_t first = out.size();
    for (const auto& t : tiles)
      for (int r = 0; r < J; ++r) {
        int lo, hi;
        range_split(0, t.n_last, r, J, 64, lo, hi);
        WorkItem it{};
        it.group = t.first;
        it.pad = t.n;
        it.region = r;
        it.nparts = J;
        if (lo == 0) {
          it.a0 = 0; it.a1 = std::min(64, hi);   // the attention-sink tile first, then newest to oldest
          it.b0 = it.a1; it.b1 = hi;
        } else {
          it.a0 = it.a1 = lo;
          it.b0 = lo; it.b1 = hi;
        }
        out.push_back(it);
      }
    longest_first(out, first);
    return J;
  };
  if (dense) {
    if (P.tiled) {
      P.J = dense_tiled_items(P.items);
    } else {
      std::vector<int64_t> lens;
      for (const auto& g : P.groups) lens.push_back(g.pos0 + g.nq);
      const int64_t chunk = split_chunk(lens);
      int J = 1;
      for (int gi = 0; gi < G; ++gi) {
        const GroupInfo& g = P.groups[gi];
        J = std::max(J, split_range(gi, 0, g.pos0 + g.nq, 0, chunk, P.items));
      }
      longest_first(P.items, 0);
      P.J = J;
    }
    P.R = P.J * P.RW;
  } else {
    // seed pass per tile: the first F keys and the last W keys of the tile's
    // last query, the window split Js ways (regions 0..Js-1) so that the
    // launch fills the GPU; the keys in between get a certificate
    int64_t loff = 0;
    int max_bounded = 0;
    // split kernel (decode-like): about half as many seed items as CUs, each a
    // window share of at least 2048 keys for its 8 wavefronts
    const int Js = P.tiled ? choose_splits(NT, std::min<int64_t>(avg_keys, P.W + P.F), tiled_target, 1024)
                           : choose_splits(NT, std::min<int64_t>(avg_keys, P.W + P.F), kSplitItems / 2, 2048);
    P.Js = Js;
    // extra seed keys: one share per 2048 listed keys of a group (list kernel,
    // one wavefront each), or one 8-wavefront item per group (split kernel)
    const int X = cfg.seed_count <= 0 ? 0
                  : (P.tiled ? (int)std::min<int64_t>(8, std::max<int64_t>(1, ((int64_t)P.QW * cfg.seed_count + 2047) / 2048))
                             : 1);
    P.X = X;
    P.x_stride = ((int64_t)P.QW * cfg.seed_count + 15) / 16 * 16;
    std::vector<WorkItem> seed_extra;   // split kernel: the seed window of a tile's other groups
    for (const auto& t : tiles) {
      const int wlo = std::max(0, t.n_last - P.W);
      const int f = std::min(P.F, wlo);
      for (int r = 0; r < Js; ++r) {
        int lo, hi;
        range_split(wlo, t.n_last, r, Js, 64, lo, hi);
        WorkItem it{};
        it.group = t.first;
        it.pad = t.n;
        it.region = r;
        it.nparts = Js;
        it.a0 = 0; it.a1 = (r == 0) ? f : 0;
        it.b0 = lo; it.b1 = hi;
        it.gather = 0;
        P.seed_items.push_back(it);
        for (int i = 1; !P.tiled && i < t.n; ++i) {
          it.group = t.first + i;
          it.pad = 1;
          seed_extra.push_back(it);
        }
      }
      for (int i = 0; i < t.n; ++i) {
        GroupInfo& g = P.groups[t.first + i];
        g.bound_lo = f;
        g.n_bounded = wlo - f;
        g.list_off = loff;
        g.list_cap = (g.n_bounded + 15) / 16 * 16;
        if (!P.tiled) loff += g.list_cap;   // a list of its own per group
        max_bounded = std::max(max_bounded, g.n_bounded);
      }
      // calls with query tiles: one list area per tile, for its union list or
      // its groups' lists one after the other (compaction takes that route only
      // when they total fewer entries than the union, unless DOSA_GROUP_LISTS
      // sends every tile there: then each group has room for all its keys)
      if (P.tiled)
        loff += (cfg.flags & DOSA_GROUP_LISTS) ? (int64_t)t.n * ((wlo - f + 15) / 16 * 16 + 16)
                                               : (int64_t)(wlo - f + 15) / 16 * 16 + 16 * t.n;
    }
    // survivor lists: J shares per group (one wavefront each with the list
    // kernel; with the split kernel, 8 wavefronts each, so fewer shares)
    const int J = cfg.key_splits > 0 ? cfg.key_splits
                  : (P.tiled ? choose_splits(G, avg_keys, 2048, 1024)
                             : (int)std::max<int64_t>(1, std::min<int64_t>(16, (kSplitItems + G - 1) / std::max(G, 1))));
    P.seed_items.insert(P.seed_items.end(), seed_extra.begin(), seed_extra.end());
    // union lists of tiles (tiled kernel): up to Ju shares per tile, enough
    // workgroups to fill the GPU when every tile takes this route
    int Ju = 1;
    if (P.tiled) {
      int64_t bsum_t = 0;
      for (const auto& t : tiles) bsum_t += P.groups[t.first].n_bounded;
      Ju = cfg.key_splits > 0 ? cfg.key_splits
                              : choose_splits(NT, NT ? bsum_t / NT : 0, 4 * tiled_target, kUnionMinShare);
    }
    P.J = std::max(J, Ju);
    // calls without tiles: groups of tiles whose certificate prunes little
    // walk the whole bounded range (split kernel, balanced key ranges)
    if (!P.tiled) {
      std::vector<int64_t> lens;
      for (const auto& g : P.groups) lens.push_back(std::max(g.n_bounded, 0));
      const int64_t chunk = split_chunk(lens);
      for (int gi = 0; gi < G; ++gi) {
        const GroupInfo& g = P.groups[gi];
        if (g.n_bounded <= 0) continue;
        P.J = std::max(P.J, split_range(gi, g.bound_lo, g.bound_lo + g.n_bounded, Js + X, chunk, P.surv_tiled_items));
      }
      longest_first(P.surv_tiled_items, 0);
    }
    P.R = (Js + X + P.J) * P.RW;
    // calls with tiles: share r of Ju of the tile's union survivor list
    for (const auto& t : tiles) {
      if (!P.tiled) break;
      for (int r = 0; r < Ju; ++r) {
        WorkItem it{};
        it.group = t.first;
        it.pad = t.n;
        it.region = Js + X + r;
        it.gather = 1;
        it.a0 = r;
        it.a1 = Ju;
        P.surv_tiled_items.push_back(it);
      }
    }
    // everything else: one wavefront per group over its compacted survivor list
    for (int gi = 0; gi < G; ++gi)
      for (int r = 0; r < J; ++r) {
        WorkItem it{};
        it.group = gi;
        it.region = Js + X + r;
        it.gather = 1;
        it.a0 = r;
        it.a1 = J;
        P.surv_list_items.push_back(it);
      }
    // extra seed keys: share r of X of each group's list
    for (int gi = 0; X > 0 && gi < G; ++gi) {
      if (P.groups[gi].n_bounded <= 0) continue;
      for (int r = 0; r < X; ++r) {
        WorkItem it{};
        it.group = gi;
        it.region = Js + r;
        it.gather = 1;
        it.a0 = r;
        it.a1 = X;
        P.x_items.push_back(it);
      }
    }
    P.items = P.seed_items;
    // bound pass over LDS key tiles when tiles hold enough groups: one item per
    // (tile, 64-key-aligned share of its bounded range)
    // A bound workgroup takes 4/QW consecutive tiles of one sequence with the
    // same first bounded key, so its wavefronts hold 4 queries each; its key
    // range runs to the longest of their bounded ranges.
    auto make_bound_items = [&](const std::vector<GroupInfo>& gs, std::vector<WorkItem>& out) {
      struct BlockInfo { int first, n, lo, hi; };
      std::vector<BlockInfo> blocks;
      for (size_t ti = 0; ti < tiles.size(); ++ti) {
        const TileInfo& t = tiles[ti];
        const GroupInfo& g = gs[t.first];
        const int lo = g.bound_lo, hi = g.bound_lo + g.n_bounded;
        if (!blocks.empty()) {
          BlockInfo& bk = blocks.back();
          const GroupInfo& h = gs[bk.first];
          if (h.seq == g.seq && h.bound_lo == lo && bk.n + t.n <= TW * P.bound_gpw &&
              bk.first + bk.n == t.first) {
            bk.n += t.n;
            bk.hi = std::max(bk.hi, hi);
            continue;
          }
        }
        blocks.push_back({t.first, t.n, lo, hi});
      }
      const int NB = (int)blocks.size();
      int64_t bsum_t = 0;
      for (const auto& bk : blocks) bsum_t += bk.hi - bk.lo;
      const int Jb = choose_splits(NB, NB ? bsum_t / NB : 0, 4 * tiled_target, 2048);
      const size_t first = out.size();
      for (const auto& bk : blocks) {
        for (int r = 0; r < Jb; ++r) {
          int lo, hi;
          range_split(bk.lo, bk.hi, r, Jb, 64, lo, hi);
          if (hi <= lo && r > 0) continue;
          WorkItem it{};
          it.group = bk.first;
          it.pad = bk.n;
          it.a0 = lo; it.a1 = hi;
          it.b0 = r;
          out.push_back(it);
        }
      }
      longest_first(out, first);
    };
    if (P.tiled) {
      P.bound_gpw = 4 / P.QW;
      P.two_rounds = (cfg.flags & DOSA_TWO_ROUNDS) != 0;
      if (!P.two_rounds) {
        make_bound_items(P.groups, P.bound_items);
      } else {
        // Two rounds: round 1 bounds the newer half of each tile's bounded
        // range with the seed threshold and scores its survivors; the K-th
        // largest exact score of the seed and round-1 candidates then becomes
        // the threshold of round 2 over the older half.  The split is a
        // multiple of 64 keys from the range's start (the bound kernels'
        // alignment); both rounds share the tile's list area.
        P.groups_r1 = P.groups;
        P.groups_r2 = P.groups;
        for (int gi = 0; gi < G; ++gi) {
          const GroupInfo& g = P.groups[gi];
          const int half = g.n_bounded > 0 ? (g.n_bounded / 2) / 64 * 64 : 0;
          P.groups_r1[gi].bound_lo = g.bound_lo + half;
          P.groups_r1[gi].n_bounded = g.n_bounded - half;
          P.groups_r2[gi].n_bounded = half;
        }
        make_bound_items(P.groups_r1, P.bound_items);
        make_bound_items(P.groups_r2, P.bound_items2);
        for (WorkItem it : P.surv_tiled_items) {
          it.region += P.J;
          P.surv_tiled_items2.push_back(it);
        }
        for (WorkItem it : P.surv_list_items) {
          it.region += P.J;
          P.surv_list_items2.push_back(it);
        }
        P.R = (Js + X + 2 * P.J) * P.RW;
      }
    }
    // probe: with enough tiles, the last tile (longest contexts) is planned
    // first; if its certificate can prune no query, the call scores every
    // tile densely with the dense path's items (regions 0..Jd-1).  Calls
    // without tiles (decode-like: every sequence a tile of its own) plan
    // their groups in the probe -- up to kProbeGroups of them, one launch of
    // one workgroup per query -- and score densely with the dense path's
    // balanced split items.
    if (NT >= 8 && (cfg.flags & DOSA_NO_PROBE) == 0) {
      P.probe = true;
      if (P.tiled) {
        const TileInfo& t = tiles.back();
        P.probe_group = t.first;
        P.probe_ngroups = t.n;
        P.probe_q0 = P.groups[t.first].q_row0;
        P.probe_nq = 0;
        for (int i = 0; i < t.n; ++i) P.probe_nq += P.groups[t.first + i].nq;
        P.Jd = dense_tiled_items(P.dense_items);
      } else {
        // at most kProbeGroups groups (the last ones): the decision needs a
        // sample, and the plan launch's time grows with its rounds of workgroups
        P.probe_ngroups = std::min(G, kProbeGroups);
        P.probe_group = G - P.probe_ngroups;
        P.probe_q0 = P.groups[P.probe_group].q_row0;
        P.probe_nq = 0;
        for (int gi = P.probe_group; gi < G; ++gi) P.probe_nq += P.groups[gi].nq;
        std::vector<int64_t> lens;
        for (const auto& g : P.groups) lens.push_back(g.pos0 + g.nq);
        const int64_t chunk = split_chunk(lens);
        P.Jd = 1;
        for (int gi = 0; gi < G; ++gi) {
          const GroupInfo& g = P.groups[gi];
          P.Jd = std::max(P.Jd, split_range(gi, 0, g.pos0 + g.nq, 0, chunk, P.dense_items));
        }
        longest_first(P.dense_items, 0);
      }
      P.R = std::max(P.R, P.Jd * P.RW);
    }
    P.items.insert(P.items.end(), P.surv_tiled_items.begin(), P.surv_tiled_items.end());
    P.items.insert(P.items.end(), P.surv_list_items.begin(), P.surv_list_items.end());
    P.items.insert(P.items.end(), P.bound_items.begin(), P.bound_items.end());
    P.items.insert(P.items.end(), P.dense_items.begin(), P.dense_items.end());
    P.items.insert(P.items.end(), P.bound_items2.begin(), P.bound_items2.end());
    P.items.insert(P.items.end(), P.surv_tiled_items2.begin(), P.surv_tiled_items2.end());
    P.items.insert(P.items.end(), P.surv_list_items2.begin(), P.surv_list_items2.end());
    P.items.insert(P.items.end(), P.x_items.begin(), P.x_items.end());
    P.list_total = loff;
    P.mask_words = (max_bounded + 63) / 64;
    int64_t bsum = 0;
    for (auto& g : P.groups) bsum += g.n_bounded;
    P.bound_splits = choose_splits(G, G ? bsum / G : 0, 4096, 4096);
  }
  // Candidate region capacity.  A region scoring n keys against a running
  // threshold receives about K (1 + ln(n / K)) entries (the expected number of
  // records among n draws); automatic sizing takes 1.3x that plus slack, so a
  // region rarely has to be compacted mid-sweep, and never more than n + 64.
  const size_t n_main_items = P.items.size();
  const size_t x_end = n_main_items, x_begin = x_end - P.x_items.size();   // extra seed items come last
  auto est_cap = [&](int64_t max_n) {
    const double k = (double)topk;
    const double est = 1.3 * k * (1.0 + std::log(std::max((double)max_n, k) / k)) + 256.0;
    int64_t cap = std::min<int64_t>((int64_t)est, max_n + 64);
    cap = std::max<int64_t>(cap, topk + 64);
    return (int)((cap + 63) / 64 * 64);
  };
  if (cfg.buffer_cap == 0) {
    int64_t max_n = 0;
    for (size_t ii = 0; ii < n_main_items; ++ii) {
      const WorkItem& it = P.items[ii];
      int64_t n = (int64_t)(it.a1 - it.a0) + (it.b1 - it.b0);
      if (it.gather) {
        const int64_t nb = P.groups[it.group].n_bounded;
        n = std::max<int64_t>((nb + it.a1 - 1) / it.a1, std::min<int64_t>(nb, 2 * kUnionMinShare)) + 64;
        if (ii >= x_begin && ii < x_end) n = std::min<int64_t>(nb, (P.x_stride + it.a1 - 1) / it.a1) + 64;
      }
      // split kernel: each wavefront's region takes every 8th 64-key step
      if (P.RW > 1) n = ((n + 63) / 64 + P.RW - 1) / P.RW * 64;
      max_n = std::max(max_n, n);
    }
    P.cap = est_cap(max_n);
  } else {
    P.cap = (cfg.buffer_cap + 63) / 64 * 64;
  }
  // workspace layout
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  P.o_groups = take(sizeof(GroupInfo) * std::max(G, 1));
  P.o_items = take(sizeof(WorkItem) * std::max<size_t>(P.items.size(), 1));
  if (!dense) P.o_seqinfo = take((size_t)2 * (batch + 1) * sizeof(int32_t));   // cu_kv, cu_blk: copied with the plan
  if (P.two_rounds) {   // the two rounds' group tables, copied with the plan too
    P.o_groups1 = take(sizeof(GroupInfo) * std::max(G, 1));
    P.o_groups2 = take(sizeof(GroupInfo) * std::max(G, 1));
  }
  P.o_cand = take((size_t)P.total_q * P.R * P.cap * sizeof(u64));
  P.o_counts = take((size_t)P.total_q * P.R * sizeof(uint32_t));
  const int LS = 16 / P.QW;   // weighted-query terms per query
  P.o_lrows = take((size_t)P.total_q * LS * d * qbytes(q_dtype));
  P.o_lsig = take((size_t)P.total_q * LS * sizeof(float));
  P.o_lerr = take((size_t)P.total_q * 2 * sizeof(float));
  P.o_tshare = take((size_t)P.total_q * sizeof(uint32_t));
  // split thresholds: the dense launch's J parts; in the pruned path the seed
  // launch's Js parts, then the dense launch's Jd (calls with a probe) or the
  // survivor range items' J (calls without tiles)
  P.n_parts = dense ? P.J : P.Js + (P.probe ? P.Jd : 0) + (P.tiled ? 0 : P.J);
  if (P.n_parts > 0) P.o_tpart = take((size_t)P.total_q * P.n_parts * sizeof(uint32_t));
  if (!dense) {
    P.o_tau = take((size_t)P.total_q * sizeof(float));
    P.o_rows = take((size_t)P.total_q * 4 * d * qbytes(q_dtype));
    P.o_coef = take((size_t)P.total_q * kCoefStride * sizeof(float));
    P.o_norms = take((size_t)std::max<int64_t>(P.total_k, 1) * sizeof(float));
    P.o_flag = take(2 * sizeof(int32_t));   // prunes flag, probe ticket
    P.o_masks = take((size_t)std::max(G, 1) * std::max(P.mask_words, 1) * sizeof(u64));
    P.o_lists = take((size_t)std::max<int64_t>(P.list_total, 1) * sizeof(int32_t));
    P.o_listlen = take((size_t)std::max(G, 1) * sizeof(int32_t));
    P.o_liststart = take((size_t)std::max(G, 1) * sizeof(int32_t));
    P.o_gflags = take((size_t)std::max(G, 1) * sizeof(int32_t));
    if (P.X > 0) {
      P.o_xlists = take((size_t)std::max(G, 1) * P.x_stride * sizeof(int32_t));
      P.o_xlen = take((size_t)std::max(G, 1) * sizeof(int32_t));
    }
    P.o_mode = take(sizeof(int32_t));
    P.o_order = take(sizeof(int32_t) * std::max<size_t>(P.surv_tiled_items.size(), 1));
    const int kbytes = (k_dtype == DOSA_F32) ? 4 : (k_dtype == DOSA_BF16 ? 2 : 1);
    P.o_blk_code = take((size_t)std::max<int64_t>(P.n_blocks, 1) * d * kbytes);
    P.o_blk_info = take((size_t)std::max<int64_t>(P.n_blocks, 1) * 4 * sizeof(float));
  }
  P.total = o;
}

bool valid_ptrs(const void* q, const float* q_scale, const float* w, const void* k, const float* k_scale,
                int32_t q_dtype, int32_t k_dtype, const int32_t* page_table, int32_t page_size,
                int32_t max_pages, int32_t* out_idx, int64_t total_q) {
  if (total_q > 0 && (q == nullptr || w == nullptr || k == nullptr || out_idx == nullptr)) return false;
  if (total_q > 0 && q_dtype == DOSA_FP8_E4M3FN && q_scale == nullptr) return false;
  if (total_q > 0 && k_dtype == DOSA_FP8_E4M3FN && k_scale == nullptr) return false;
  if (page_table != nullptr && (page_size <= 0 || (page_size % 16) != 0 || max_pages <= 0)) return false;
  return true;
}

int run(bool dense, const void* q, int32_t q_dtype, const float* q_scale, const float* w, const void* k,
        int32_t k_dtype, const float* k_scale, const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
        const int32_t* page_table, int32_t page_size, int32_t max_pages, int32_t H, int32_t d, int32_t topk,
        int32_t* out_idx, float* out_score, void* workspace, size_t workspace_bytes, const dosa_config& cfg,
        dosa_stats* stats, hipStream_t stream);

// ---------------------------------------------------------------------------
// scratch memory of dosa_indexer_topk_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it only stands in for the
// symbol); it uses the device address hipGetSymbolAddress returns, looked up
// once per device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)DOSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices) {
    g_err = "device index " + std::to_string(dev) + " out of range for the scratch table";
    return DOSA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) {
      g_err = "hipGetSymbolAddress(scratch) returned NULL";
      return DOSA_ERR_HIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return DOSA_OK;
}

}  // namespace

extern "C" {

int dosa_default_config(int32_t topk, dosa_config* cfg) {
  if (cfg == nullptr) return DOSA_ERR_INVALID_ARG;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->num_proxies = 3;
  // 4K: at K = 2048 the seed's K-th score then prunes far more than with 2K
  // seed keys (correlated-heads recipe: 21% -> 15% of bounded keys survive at
  // 128K, 23% -> 9% at 32K) for a seed pass that costs little more
  cfg->seed_window = std::max(64, 4 * topk);
  cfg->seed_prefix = 64;
  cfg->buffer_cap = 0;   // automatic
  cfg->key_splits = 0;
  cfg->neg_support_frac = 0.5f;
  cfg->flags = 0;
  cfg->debug_ub = nullptr;
  return DOSA_OK;
}

size_t dosa_workspace_size(int32_t batch, const int32_t* q_lens, const int32_t* kv_lens, int32_t H, int32_t d,
                           int32_t topk, int32_t q_dtype, int32_t k_dtype, int32_t paged, int32_t dense,
                           const dosa_config* cfg) {
  if (check_shapes(batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype) != DOSA_OK) return 0;
  dosa_config c;
  if (resolve_cfg(cfg, topk, &c) != DOSA_OK) return 0;
  Plan P;
  build_plan(P, batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype, paged != 0, dense != 0, c);
  return std::max<size_t>(P.total, 256);
}

int dsa_indexer_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w, const void* k,
                     int32_t k_dtype, const float* k_scale, const int32_t* q_lens, const int32_t* kv_lens,
                     int32_t batch, const int32_t* page_table, int32_t page_size, int32_t max_pages, int32_t H,
                     int32_t d, int32_t topk, int32_t* out_idx, float* out_score, void* workspace,
                     size_t workspace_bytes, const dosa_config* cfg, dosa_stats* stats, void* stream) {
  try {
    int st = check_shapes(batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype);
    if (st != DOSA_OK) return st;
    dosa_config c;
    st = resolve_cfg(cfg, topk, &c);
    if (st != DOSA_OK) return st;
    c.flags &= DOSA_SORTED;
    c.seed_count = 0;
    return run(true, q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, batch, page_table, page_size,
               max_pages, H, d, topk, out_idx, out_score, workspace, workspace_bytes, c, stats,
               static_cast<hipStream_t>(stream));
  } catch (...) {
    g_err = "internal error";
    return DOSA_ERR_HIP;
  }
}

int dosa_indexer_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w, const void* k,
                      int32_t k_dtype, const float* k_scale, const int32_t* q_lens, const int32_t* kv_lens,
                      int32_t batch, const int32_t* page_table, int32_t page_size, int32_t max_pages, int32_t H,
                      int32_t d, int32_t topk, int32_t* out_idx, float* out_score, void* workspace,
                      size_t workspace_bytes, const dosa_config* cfg, dosa_stats* stats, void* stream) {
  try {
    int st = check_shapes(batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype);
    if (st != DOSA_OK) return st;
    dosa_config c;
    st = resolve_cfg(cfg, topk, &c);
    if (st != DOSA_OK) return st;
    return run(false, q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, batch, page_table, page_size,
               max_pages, H, d, topk, out_idx, out_score, workspace, workspace_bytes, c, stats,
               static_cast<hipStream_t>(stream));
  } catch (...) {
    g_err = "internal error";
    return DOSA_ERR_HIP;
  }
}

int dosa_indexer_topk_noalloc(const void* q, int32_t q_dtype, const float* q_scale, const float* w, const void* k,
                              int32_t k_dtype, const float* k_scale, const int32_t* q_lens, const int32_t* kv_lens,
                              int32_t batch, const int32_t* page_table, int32_t page_size, int32_t max_pages,
                              int32_t H, int32_t d, int32_t topk, int32_t* out_idx, float* out_score,
                              const dosa_config* cfg, dosa_stats* stats, void* stream) {
  try {
    int st = check_shapes(batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype);
    if (st != DOSA_OK) return st;
    dosa_config c;
    st = resolve_cfg(cfg, topk, &c);
    if (st != DOSA_OK) return st;
    {
      Plan P;
      build_plan(P, batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype, page_table != nullptr, false, c);
      if (P.total > kScratchBytes) {
        g_err = "the call needs " + std::to_string(P.total) + " bytes of workspace; the no-allocation entry "
                "point has " + std::to_string(kScratchBytes) + " (use dosa_indexer_topk with a workspace)";
        return DOSA_ERR_UNSUPPORTED;
      }
    }
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != DOSA_OK) return st;
    return run(false, q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, batch, page_table, page_size,
               max_pages, H, d, topk, out_idx, out_score, ws, kScratchBytes, c, stats,
               static_cast<hipStream_t>(stream));
  } catch (...) {
    g_err = "internal error";
    return DOSA_ERR_HIP;
  }
}

const char* dosa_status_string(int status) {
  switch (status) {
    case DOSA_OK: return "ok";
    case DOSA_ERR_INVALID_ARG: return g_err.empty() ? "invalid argument" : g_err.c_str();
    case DOSA_ERR_UNSUPPORTED: return g_err.empty() ? "unsupported shape or dtype" : g_err.c_str();
    case DOSA_ERR_WORKSPACE: return g_err.empty() ? "workspace too small" : g_err.c_str();
    case DOSA_ERR_HIP: return g_err.empty() ? "HIP error" : g_err.c_str();
  }
  return "unknown status";
}

const char* dosa_version(void) { return "dosa-indexer 0.1 (gfx950)"; }

int dosa_profile_begin(void) {
  g_prof.on = true;
  g_prof.used = 0;
  g_prof.recs.clear();
  return DOSA_OK;
}

int dosa_profile_end(dosa_kernel_time* out, int32_t max_entries) {
  if (!g_prof.on) return 0;
  g_prof.on = false;
  double ms[P_COUNT] = {0};
  int n[P_COUNT] = {0};
  for (auto& r : g_prof.recs) {
    hipEvent_t a = g_prof.pool[r.second], b = g_prof.pool[r.second + 1];
    hipError_t e = hipEventSynchronize(b);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
    float t = 0.f;
    e = hipEventElapsedTime(&t, a, b);
    if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
    ms[r.first] += t;
    n[r.first] += 1;
  }
  g_prof.recs.clear();
  g_prof.used = 0;
  int k = 0;
  for (int i = 0; i < P_COUNT; ++i) {
    if (n[i] == 0) continue;
    if (out != nullptr && k < max_entries) {
      out[k].name = kPassNames[i];
      out[k].launches = n[i];
      out[k].total_ms = ms[i];
    }
    ++k;
  }
  return std::min(k, max_entries);
}

}  // extern "C"

namespace {

int run(bool dense, const void* q, int32_t q_dtype, const float* q_scale, const float* w, const void* k,
        int32_t k_dtype, const float* k_scale, const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
        const int32_t* page_table, int32_t page_size, int32_t max_pages, int32_t H, int32_t d, int32_t topk,
        int32_t* out_idx, float* out_score, void* workspace, size_t workspace_bytes, const dosa_config& cfg,
        dosa_stats* stats, hipStream_t stream) {
  Plan P;
  build_plan(P, batch, q_lens, kv_lens, H, d, topk, q_dtype, k_dtype, page_table != nullptr, dense, cfg);
  if (!valid_ptrs(q, q_scale, w, k, k_scale, q_dtype, k_dtype, page_table, page_size, max_pages, out_idx,
                  P.total_q)) {
    g_err = "null input/output pointer, missing fp8 scale or bad page geometry";
    return DOSA_ERR_INVALID_ARG;
  }
  if (workspace == nullptr || workspace_bytes < P.total) {
    g_err = "workspace needs " + std::to_string(P.total) + " bytes";
    return DOSA_ERR_WORKSPACE;
  }
  if (P.total_q == 0) return DOSA_OK;
  char* ws = static_cast<char*>(workspace);
  unsigned long long* st = reinterpret_cast<unsigned long long*>(stats);
  hipError_t e;
  // The call's plan -- groups, work items and (pruned path) the sequences'
  // key offsets, adjacent in the workspace -- goes over in one copy: a copy
  // from pageable host memory can hold the host until the stream reaches it,
  // so one copy at the start costs one such wait instead of one per array.
  {
    const size_t n_items = sizeof(WorkItem) * P.items.size();
    const size_t end = dense ? P.o_items + n_items
                       : (P.two_rounds ? P.o_groups2 + sizeof(GroupInfo) * P.groups.size()
                                       : P.o_seqinfo + (size_t)2 * (batch + 1) * sizeof(int32_t));
    std::vector<char> stage(end - P.o_groups, 0);
    std::memcpy(stage.data(), P.groups.data(), sizeof(GroupInfo) * P.groups.size());
    std::memcpy(stage.data() + (P.o_items - P.o_groups), P.items.data(), n_items);
    if (!dense) {
      int32_t* cu = reinterpret_cast<int32_t*>(stage.data() + (P.o_seqinfo - P.o_groups));
      int32_t* cub = cu + (batch + 1);
      cu[0] = 0;
      cub[0] = 0;
      for (int b = 0; b < batch; ++b) {
        cu[b + 1] = cu[b] + kv_lens[b];
        cub[b + 1] = cub[b] + (kv_lens[b] + kKeyBlock - 1) / kKeyBlock;
      }
      if (P.two_rounds) {
        std::memcpy(stage.data() + (P.o_groups1 - P.o_groups), P.groups_r1.data(), sizeof(GroupInfo) * P.groups.size());
        std::memcpy(stage.data() + (P.o_groups2 - P.o_groups), P.groups_r2.data(), sizeof(GroupInfo) * P.groups.size());
      }
    }
    e = hipMemcpyAsync(ws + P.o_groups, stage.data(), stage.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(plan)");
  }
  if (st) {
    unsigned long long add[12] = {P.pairs_total, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    e = launch_stats_add(st, add, stream);
    if (e != hipSuccess) return fail_hip(e, "stats");
  }
  int page_shift = -1;
  if (page_table != nullptr && (page_size & (page_size - 1)) == 0)
    for (page_shift = 0; (1 << page_shift) < page_size; ++page_shift) {}
  Inputs in{q, q_scale, w, k, k_scale, page_table, page_size, max_pages, H, page_shift};
  PrepLaunch pr{q, w, H, P.total_q, ws + P.o_lrows, reinterpret_cast<float*>(ws + P.o_lsig),
                reinterpret_cast<float*>(ws + P.o_lerr), dense ? nullptr : reinterpret_cast<int32_t*>(ws + P.o_flag),
                reinterpret_cast<uint32_t*>(ws + P.o_tshare),
                P.n_parts > 0 ? reinterpret_cast<uint32_t*>(ws + P.o_tpart) : nullptr, P.n_parts,
                reinterpret_cast<uint32_t*>(ws + P.o_counts), P.R};
  uint32_t* tshare = kShareTheta ? reinterpret_cast<uint32_t*>(ws + P.o_tshare) : nullptr;
  uint32_t* tpart = P.n_parts > 0 ? reinterpret_cast<uint32_t*>(ws + P.o_tpart) : nullptr;
  {
    PassScope ps(P_PREP, stream);
    e = launch_prep(P.combo, H, d, pr, stream);
  }
  if (e != hipSuccess) return fail_hip(e, "prep kernel launch");
  CandBuf cb{reinterpret_cast<u64*>(ws + P.o_cand), reinterpret_cast<uint32_t*>(ws + P.o_counts), P.R, P.cap,
             (int64_t)P.total_q};
  const GroupInfo* dg = reinterpret_cast<const GroupInfo*>(ws + P.o_groups);
  const WorkItem* di = reinterpret_cast<const WorkItem*>(ws + P.o_items);
  if (dense) {
    ScoreLaunch sl{};
    sl.theta_share = tshare;
    sl.in = in;
    sl.lrows = pr.rows;
    sl.lsig = pr.sig;
    sl.groups = dg;
    sl.items = di;
    sl.n_items = (int)P.items.size();
    sl.cb = cb;
    sl.theta_init = nullptr;
    sl.topk = topk;
    sl.stats = st;
    sl.scored_slot = 4;
    sl.tiled = P.tiled ? 1 : 2;
    sl.role = ROLE_DENSE;
    sl.theta_part = tpart;
    sl.part_stride = P.n_parts;
    {
      PassScope ps(P_SCORE_DENSE, stream);
      e = launch_score(P.combo, H, d, sl, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "score kernel launch");
  } else {
    const int G = (int)P.groups.size();
    int32_t max_kv = 0;
    for (int b = 0; b < batch; ++b) max_kv = std::max(max_kv, kv_lens[b]);
    int32_t* cu_dev = reinterpret_cast<int32_t*>(ws + P.o_seqinfo);
    float* tau = reinterpret_cast<float*>(ws + P.o_tau);
    float* norms = reinterpret_cast<float*>(ws + P.o_norms);
    float* coef = reinterpret_cast<float*>(ws + P.o_coef);
    u64* masks = reinterpret_cast<u64*>(ws + P.o_masks);
    int32_t* lists = reinterpret_cast<int32_t*>(ws + P.o_lists);
    int32_t* list_len = reinterpret_cast<int32_t*>(ws + P.o_listlen);
    int32_t* gflags = reinterpret_cast<int32_t*>(ws + P.o_gflags);
    int32_t* prunes = reinterpret_cast<int32_t*>(ws + P.o_flag);   // cleared by the prep kernel
    // device item order (the order of P.items): seed, tiled survivors, list survivors, bound,
    // dense, round-2 bound, round-2 tiled survivors, round-2 list survivors, extra seed
    const size_t off_surv = P.seed_items.size(), off_list = off_surv + P.surv_tiled_items.size(),
                 off_bound = off_list + P.surv_list_items.size(), off_dense = off_bound + P.bound_items.size(),
                 off_bound2 = off_dense + P.dense_items.size(), off_surv2 = off_bound2 + P.bound_items2.size(),
                 off_list2 = off_surv2 + P.surv_tiled_items2.size(),
                 off_x = off_list2 + P.surv_list_items2.size();
    int32_t* mode = P.probe ? reinterpret_cast<int32_t*>(ws + P.o_mode) : nullptr;
    // 1b. probe: plan of the last tile only, with a threshold estimated from
    //     the plan's sample of seed-window keys, then the decision whether the
    //     call runs the certificate pipeline or dense scoring
    int32_t* list_start = reinterpret_cast<int32_t*>(ws + P.o_liststart);
    if (P.probe) {
      PassScope ps(P_PROBE, stream);
      PlanLaunch pp{};
      pp.in = in;
      pp.groups = dg + P.probe_group;
      pp.n_groups = P.probe_ngroups;
      pp.num_proxies = cfg.num_proxies;
      pp.seed_window = P.W;
      pp.neg_frac = cfg.neg_support_frac;
      pp.flags = cfg.flags;
      pp.tau = nullptr;                // threshold estimated from the sampled window keys
      pp.topk = topk;
      pp.seed_prefix = P.F;
      pp.lerr = pr.err;
      pp.prunes = prunes;
      pp.rows = ws + P.o_rows;
      pp.coef = coef;
      pp.ticket = prunes + 1;
      pp.decide_nq = P.probe_nq;
      pp.decide_mode = mode;
      pp.stats = st;
      e = launch_plan(P.combo, H, d, pp, stream);
      if (e != hipSuccess) return fail_hip(e, "probe plan kernel launch");
    }
    // With a probe, the certificate stages (steps 2-7) go to the side stream
    // and the dense alternative (step 8) stays on the caller's stream, when
    // the dense alternative runs in at most two workgroups per CU: its
    // workgroups then finish together and the certificate launches (which
    // return at once after a dense decision) run in its tail.  With more
    // rounds of dense workgroups, the certificate launches' empty workgroups
    // (tens of thousands at a 32K-query call) interleave with them and cost
    // more than the serial launches (32K bf16 prefill: 11.8 against 9.1 ms).
    SideFork sf;
    hipStream_t cs = stream;
    // Calls without tiles stay on one stream too: the split kernel's
    // workgroups each take a whole CU, and the side stream's empty workgroups
    // (thousands, across eight launches) hold CUs it waits for (decode batch:
    // 1.28 ms on two streams, see the measurements).
    // Small calls (fewer than kSideStreamMinPairs causal pairs) stay on one
    // stream as well: their launches are short, and the fork and join cost
    // more than the overlap saves (tiny prefill: 0.5-0.9 ms on two streams
    // from run to run, 0.49 ms on one).
    if (P.probe && P.tiled && P.dense_items.size() <= (size_t)kSideStreamMaxItems &&
        P.pairs_total >= kSideStreamMinPairs) {
      e = sf.open(stream);
      if (e != hipSuccess) return fail_hip(e, "side stream");
      if (sf.side != nullptr) cs = sf.side;
    }
    // 2. seed pass: exact scores of the seed keys into regions 0..Js-1
    ScoreLaunch sl{};
    sl.theta_share = tshare;
    sl.mode = mode;
    sl.run_if = MODE_PRUNED;
    sl.in = in;
    sl.lrows = pr.rows;
    sl.lsig = pr.sig;
    sl.groups = dg;
    sl.items = di;
    sl.n_items = (int)P.seed_items.size();
    sl.cb = cb;
    sl.topk = topk;
    sl.stats = st;
    sl.scored_slot = 1;
    sl.tiled = P.tiled ? 1 : 2;
    sl.role = ROLE_SEED;
    sl.theta_part = tpart;
    sl.part_stride = P.n_parts;
    {
      PassScope ps(P_SCORE_SEED, cs);
      e = launch_score(P.combo, H, d, sl, cs);
    }
    if (e != hipSuccess) return fail_hip(e, "seed score kernel launch");
    // 2b. extra seed keys: the union list of each group, scored into regions
    //     Js..Js+X-1 (read by the threshold select only; compaction clears them)
    if (P.X > 0) {
      PassScope ps(P_SEED_EXTRA, cs);
      int32_t* xlists = reinterpret_cast<int32_t*>(ws + P.o_xlists);
      int32_t* xlen = reinterpret_cast<int32_t*>(ws + P.o_xlen);
      SeedUnionLaunch su{dg, G, cfg.seed_idx, cfg.seed_count, xlists, P.x_stride, xlen, mode, MODE_PRUNED};
      e = launch_seed_union(su, cs);
      if (e == hipSuccess && !P.x_items.empty()) {
        ScoreLaunch xl{};
        xl.theta_share = tshare;
        xl.mode = mode;
        xl.run_if = MODE_PRUNED;
        xl.in = in;
        xl.lrows = pr.rows;
        xl.lsig = pr.sig;
        xl.groups = dg;
        xl.items = di + off_x;
        xl.n_items = (int)P.x_items.size();
        xl.cb = cb;
        xl.lists = xlists;
        xl.list_len = xlen;
        xl.list_stride = P.x_stride;
        xl.topk = topk;
        xl.stats = st;
        xl.scored_slot = 1;
        xl.tiled = P.tiled ? 0 : 2;
        xl.role = ROLE_SURVIVORS;
        e = launch_score(P.combo, H, d, xl, cs);
      }
    }
    if (e != hipSuccess) return fail_hip(e, "extra seed kernel launch");
    // 3. tau = K-th largest seed score
    SelectLaunch ts{};
    ts.mode = mode;
    ts.run_if = MODE_PRUNED;
    ts.cb = cb;
    ts.total_q = (int32_t)P.total_q;
    ts.topk = topk;
    ts.r0 = 0;
    ts.r1 = (P.Js + P.X) * P.RW;
    ts.tau_out = tau;
    ts.tau_copy = cfg.debug_tau;
    {
      PassScope ps(P_SELECT_SEED, cs);
      e = launch_select(ts, cs);
    }
    if (e != hipSuccess) return fail_hip(e, "seed select kernel launch");
    // 4. certificate plan per query
    PlanLaunch pl{};
    pl.mode = mode;
    pl.run_if = MODE_PRUNED;
    pl.in = in;
    pl.groups = dg;
    pl.n_groups = G;
    pl.num_proxies = cfg.num_proxies;
    pl.seed_window = P.W;
    pl.neg_frac = cfg.neg_support_frac;
    pl.flags = cfg.flags;
    pl.tau = tau;
    pl.lerr = pr.err;
    pl.prunes = prunes;
    pl.rows = ws + P.o_rows;
    pl.coef = coef;
    {
      PassScope ps(P_PLAN, cs);
      e = launch_plan(P.combo, H, d, pl, cs);
    }
    if (e != hipSuccess) return fail_hip(e, "plan kernel launch");
    // 4b. per-key norms for the bound pass; the launch returns at once when the
    //     plan found no query whose certificate can prune
    const bool key_blocks = P.tiled && (cfg.flags & DOSA_KEY_BLOCKS) != 0;
    NormLaunch nl{in, cu_dev, batch, P.total_k, max_kv, norms, cfg.debug_ub != nullptr ? nullptr : prunes,
                  cu_dev + (batch + 1), key_blocks ? reinterpret_cast<uint8_t*>(ws + P.o_blk_code) : nullptr,
                  reinterpret_cast<float*>(ws + P.o_blk_info)};
    {
      PassScope ps(P_NORMS, cs);
      e = launch_key_norms(P.combo, d, nl, cs);
      if (e == hipSuccess) e = launch_key_blocks(P.combo, d, nl, cs);
    }
    if (e != hipSuccess) return fail_hip(e, "key norm kernel launch");
    // 5.-7. bound pass, compaction and survivor scoring: one round over every
    //    bounded key, or (two rounds) the newer half of each tile's bounded
    //    range, a raised threshold, then the older half
    auto round = [&](const GroupInfo* rg, size_t boff, size_t nb, size_t soff, size_t ns, size_t loff, size_t nl,
                     int r0, int r1, bool first) -> int {
      // 5. bound pass -> survivor bitmasks
      BoundLaunch bl{};
      bl.mode = mode;
      bl.run_if = MODE_PRUNED;
      bl.in = in;
      bl.groups = rg;
      bl.n_groups = G;
      bl.rows = ws + P.o_rows;
      bl.coef = coef;
      bl.norms = norms;
      bl.masks = masks;
      bl.mask_words = std::max(P.mask_words, 1);
      bl.debug_ub = cfg.debug_ub;
      bl.debug_ld = max_kv;
      bl.debug_mask = reinterpret_cast<unsigned long long*>(cfg.debug_mask);
      bl.debug_mask_ld = (max_kv + 63) / 64;
      if (key_blocks) {
        bl.blk_code = reinterpret_cast<const uint8_t*>(ws + P.o_blk_code);
        bl.blk_info = reinterpret_cast<const float*>(ws + P.o_blk_info);
      }
      bl.splits = P.bound_splits;
      bl.count_skipped = first ? 1 : 0;
      if (nb > 0) {
        bl.items = di + boff;
        bl.n_items = (int)nb;
        bl.groups_per_wave = P.bound_gpw;
      }
      bl.stats = st;
      {
        PassScope ps(P_BOUND, cs);
        e = launch_bound(P.combo, H, d, bl, cs);
      }
      if (e != hipSuccess) return fail_hip(e, "bound kernel launch");
      // 6. compaction -> survivor key lists
      CompactLaunch cl{};
      cl.groups = rg;
      cl.tiles = di;                    // the seed items: Js per tile, the first names the tile
      cl.tile_stride = P.Js;
      cl.n_tiles = P.n_tiles;
      cl.allow_union = P.tiled ? 1 : 0;
      cl.force_lists = (cfg.flags & DOSA_GROUP_LISTS) ? 1 : 0;
      cl.coef = coef;
      cl.masks = masks;
      cl.mask_words = std::max(P.mask_words, 1);
      cl.lists = lists;
      cl.list_len = list_len;
      cl.list_start = list_start;
      cl.group_flags = gflags;
      cl.cb = cb;
      cl.r0 = r0;
      cl.r1 = r1;
      cl.mode = mode;
      cl.run_if = MODE_PRUNED;
      {
        PassScope ps(P_COMPACT, cs);
        e = launch_compact(cl, cs);
      }
      if (e != hipSuccess) return fail_hip(e, "compact kernel launch");
      // 7. survivors scored with all heads into the round's regions, threshold starts at tau:
      //    flagged tiles take the tiled kernel over their union list (or, in calls
      //    without tiles, over the bounded range), the other groups walk their own lists
      ScoreLaunch ml{};
      ml.theta_share = tshare;
      ml.mode = mode;
      ml.run_if = MODE_PRUNED;
      ml.in = in;
      ml.lrows = pr.rows;
      ml.lsig = pr.sig;
      ml.groups = rg;
      ml.cb = cb;
      ml.theta_init = tau;
      ml.lists = lists;
      ml.list_len = list_len;
      ml.list_start = list_start;
      ml.topk = topk;
      ml.stats = st;
      ml.scored_slot = 4;
      ml.tile_flags = gflags;
      ml.role = ROLE_SURVIVORS;
      {
        PassScope ps(P_SURV_TILES, cs);
        ml.items = di + soff;
        ml.n_items = (int)ns;
        ml.tiled = P.tiled ? 1 : 2;
        ml.flag_mode = 1;
        if (!P.tiled) {   // survivor range items of groups scored whole: disjoint sweeps
          ml.theta_part = tpart;
          ml.part_stride = P.n_parts;
          ml.part_base = P.Js;
          ml.part_rbase = P.Js + P.X;
        }
        // union shares are cut on the device: launch them longest first
        if (P.tiled && ml.n_items > 0 && ml.n_items <= kMaxOrderItems) {
          OrderLaunch ol{ml.items, ml.n_items, list_len, gflags, reinterpret_cast<int32_t*>(ws + P.o_order), mode,
                         MODE_PRUNED};
          e = launch_order(ol, cs);
          ml.order = ol.order;
        }
        if (e == hipSuccess) e = launch_score(P.combo, H, d, ml, cs);
      }
      if (e == hipSuccess) {
        PassScope ps(P_SURV_LISTS, cs);
        ml.theta_part = nullptr;
        ml.order = nullptr;
        ml.items = di + loff;
        ml.n_items = (int)nl;
        ml.tiled = P.tiled ? 0 : 2;
        ml.flag_mode = 2;
        ml.scored_slot2 = 8;
        e = launch_score(P.combo, H, d, ml, cs);
      }
      if (e != hipSuccess) return fail_hip(e, "survivor score kernel launch");
      return DOSA_OK;
    };
    if (!P.two_rounds) {
      const int rc = round(dg, off_bound, P.bound_items.size(), off_surv, P.surv_tiled_items.size(), off_list,
                           P.surv_list_items.size(), P.Js * P.RW, (P.Js + P.X + P.J) * P.RW, true);   // r0: the extra seed regions too
      if (rc != DOSA_OK) return rc;
    } else {
      const GroupInfo* dg1 = reinterpret_cast<const GroupInfo*>(ws + P.o_groups1);
      const GroupInfo* dg2 = reinterpret_cast<const GroupInfo*>(ws + P.o_groups2);
      int rc = round(dg1, off_bound, P.bound_items.size(), off_surv, P.surv_tiled_items.size(), off_list,
                     P.surv_list_items.size(), P.Js * P.RW, (P.Js + P.X + P.J) * P.RW, true);
      if (rc != DOSA_OK) return rc;
      // the raised threshold: K-th largest score of the seed and round-1
      // candidates (distinct keys, each exactly scored), into tau and the
      // plan's threshold slot of every query; the merged regions keep the
      // K entries at or above it
      SelectLaunch t2{};
      t2.mode = mode;
      t2.run_if = MODE_PRUNED;
      t2.cb = cb;
      t2.total_q = (int32_t)P.total_q;
      t2.topk = topk;
      t2.r0 = 0;
      t2.r1 = (P.Js + P.X + P.J) * P.RW;
      t2.tau_out = tau;
      t2.coef_tau = coef;
      {
        PassScope ps(P_SELECT_SEED, cs);
        e = launch_select(t2, cs);
      }
      if (e != hipSuccess) return fail_hip(e, "round threshold select kernel launch");
      rc = round(dg2, off_bound2, P.bound_items2.size(), off_surv2, P.surv_tiled_items2.size(), off_list2,
                 P.surv_list_items2.size(), (P.Js + P.X + P.J) * P.RW, (P.Js + P.X + 2 * P.J) * P.RW, false);
      if (rc != DOSA_OK) return rc;
    }
    // 8. the dense alternative, run only when the probe found nothing to prune
    if (P.probe) {
      ScoreLaunch dl{};
      dl.theta_share = tshare;
      dl.mode = mode;
      dl.run_if = MODE_UNPRUNED;
      dl.in = in;
      dl.lrows = pr.rows;
      dl.lsig = pr.sig;
      dl.groups = dg;
      dl.items = di + off_dense;
      dl.n_items = (int)P.dense_items.size();
      dl.cb = cb;
      dl.theta_init = nullptr;
      dl.topk = topk;
      dl.stats = st;
      dl.scored_slot = 4;
      dl.tiled = P.tiled ? 1 : 2;
      dl.role = ROLE_DENSE;
      dl.theta_part = tpart;
      dl.part_stride = P.n_parts;
      dl.part_base = P.Js;
      PassScope ps(P_SCORE_DENSE, stream);
      e = launch_score(P.combo, H, d, dl, stream);
      if (e != hipSuccess) return fail_hip(e, "dense score kernel launch");
    }
    e = sf.close();
    if (e != hipSuccess) return fail_hip(e, "side stream join");
  }
  SelectLaunch se{};
  se.cb = cb;
  se.total_q = (int32_t)P.total_q;
  se.topk = topk;
  se.r0 = 0;
  se.r1 = dense ? P.R : (P.Js + P.X + (P.two_rounds ? 2 : 1) * P.J) * P.RW;   // pruned path: seed, (cleared) extra seed, survivor regions
  se.out_idx = out_idx;
  se.out_score = out_score;
  se.tau_out = nullptr;
  se.r1_unpruned = P.probe ? P.Jd * P.RW : P.R;
  se.mode = dense ? nullptr : (P.probe ? reinterpret_cast<int32_t*>(ws + P.o_mode) : nullptr);
  se.run_if = -1;
  se.sorted = (cfg.flags & DOSA_SORTED) ? 1 : 0;
  se.stats = st;
  {
    PassScope ps(P_SELECT_FINAL, stream);
    e = launch_select(se, stream);
  }
  if (e != hipSuccess) return fail_hip(e, "select kernel launch");
  return DOSA_OK;
}

}  // namespace

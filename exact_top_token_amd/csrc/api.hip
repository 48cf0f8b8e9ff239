// C-ABI entry points: argument checks, work planning, workspace layout and
// kernel launches on the caller's stream.  No allocation, no host sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
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
              P_SCORE_DENSE, P_SELECT_FINAL, P_PREP, P_PROBE, P_COUNT };
const char* const kPassNames[P_COUNT] = {"key_norms", "score_seed", "select_seed", "plan", "bound", "compact",
                                         "score_survivor_tiles", "score_survivor_lists", "score_dense",
                                         "select_final", "prep", "probe"};

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
  std::vector<WorkItem> seed_items, surv_tiled_items, surv_list_items, bound_items, dense_items, probe_items;
  bool probe = false;                // DoSA: plan the last tile first, score densely if it cannot prune
  int probe_group = 0, probe_ngroups = 0, probe_q0 = 0, probe_nq = 0, Jd = 0, Jp = 0;
  int bound_gpw = 1;                 // query groups per wavefront of the tiled bound kernel
  bool tiled = true;
  int bound_splits = 1;
  int Js = 1;                        // DoSA: regions of the seed pass
  int mask_words = 0;
  int64_t list_total = 0;
  // workspace offsets
  size_t o_groups = 0, o_items = 0, o_cand = 0, o_counts = 0, o_tau = 0, o_rows = 0, o_coef = 0,
         o_norms = 0, o_masks = 0, o_lists = 0, o_listlen = 0, o_seqinfo = 0, o_gflags = 0, o_flag = 0,
         o_lrows = 0, o_lsig = 0, o_lerr = 0, o_mode = 0, o_tshare = 0, o_order = 0, total = 0;
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
  P.QW = queries_per_wave(P.combo, H, d);
  P.dense = dense;
  P.F = cfg.seed_prefix;
  P.W = std::max(cfg.seed_window, 64);
  const int TW = tile_waves();
  int64_t cq = 0, ck = 0;
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
      const int gi = (int)P.groups.size();
      if (tiles.empty() || tiles.back().seq != b || tiles.back().n == TW) tiles.push_back({gi, 0, 0, b});
      tiles.back().n += 1;
      tiles.back().n_last = g.pos0 + g.nq;
      P.groups.push_back(g);
    }
    pairs += (uint64_t)m * (uint64_t)(n - m + 1) + (uint64_t)m * (uint64_t)(m - 1) / 2;
    cq += m;
    ck += n;
  }
  for (auto& t : tiles)
    for (int i = 0; i < t.n; ++i) {
      P.groups[t.first + i].tile_first = t.first;
      P.groups[t.first + i].tile_n = t.n;
    }
  P.total_q = cq;
  P.total_k = ck;
  P.pairs_total = pairs;
  const int G = (int)P.groups.size();
  const int NT = (int)tiles.size();
  int64_t key_sum = 0;
  for (auto& t : tiles) key_sum += t.n_last;
  const int64_t avg_keys = NT ? key_sum / NT : 0;
  // Tiles that hold few groups waste the tiled kernel's wavefronts: use one
  // wavefront per group there (decode-like batches).
  P.tiled = (NT > 0) && (2 * G >= TW * NT);
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
      int J = cfg.key_splits > 0 ? cfg.key_splits : choose_splits(G, avg_keys, 2048, 1024);
      P.J = J;
      for (int gi = 0; gi < G; ++gi) {
        const GroupInfo& g = P.groups[gi];
        const int n = g.pos0 + g.nq;
        for (int r = 0; r < J; ++r) {
          int lo, hi;
          range_split(0, n, r, J, 16, lo, hi);
          WorkItem it{};
          it.group = gi;
          it.region = r;
          if (lo == 0) {
            it.a0 = 0; it.a1 = std::min(16, hi);
            it.b0 = it.a1; it.b1 = hi;
          } else {
            it.a0 = it.a1 = lo;
            it.b0 = lo; it.b1 = hi;
          }
          P.items.push_back(it);
        }
      }
    }
    P.R = P.J;
  } else {
    // seed pass per tile: the first F keys and the last W keys of the tile's
    // last query, the window split Js ways (regions 0..Js-1) so that the
    // launch fills the GPU; the keys in between get a certificate
    int64_t loff = 0;
    int max_bounded = 0;
    const int Js = choose_splits(NT, std::min<int64_t>(avg_keys, P.W + P.F), tiled_target, 1024);
    P.Js = Js;
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
        it.a0 = 0; it.a1 = (r == 0) ? f : 0;
        it.b0 = lo; it.b1 = hi;
        it.gather = 0;
        P.seed_items.push_back(it);
      }
      for (int i = 0; i < t.n; ++i) {
        GroupInfo& g = P.groups[t.first + i];
        g.bound_lo = f;
        g.n_bounded = wlo - f;
        g.list_off = (int32_t)loff;
        g.list_cap = (g.n_bounded + 15) / 16 * 16;
        loff += g.list_cap;
        max_bounded = std::max(max_bounded, g.n_bounded);
      }
    }
    const int J = cfg.key_splits > 0 ? cfg.key_splits : choose_splits(G, avg_keys, 2048, 1024);
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
    P.R = Js + P.J;
    // calls without tiles: groups of tiles whose certificate prunes little
    // walk the whole bounded range (one wavefront per group)
    if (!P.tiled) {
      for (int gi = 0; gi < G; ++gi) {
        const GroupInfo& g = P.groups[gi];
        for (int r = 0; r < J; ++r) {
          int lo, hi;
          range_split(g.bound_lo, g.bound_lo + g.n_bounded, r, J, 16, lo, hi);
          WorkItem it{};
          it.group = gi;
          it.region = Js + r;
          it.a0 = it.a1 = lo;
          it.b0 = lo; it.b1 = hi;
          P.surv_tiled_items.push_back(it);
        }
      }
    }
    // calls with tiles: share r of Ju of the tile's union survivor list
    for (const auto& t : tiles) {
      if (!P.tiled) break;
      for (int r = 0; r < Ju; ++r) {
        WorkItem it{};
        it.group = t.first;
        it.pad = t.n;
        it.region = Js + r;
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
        it.region = Js + r;
        it.gather = 1;
        it.a0 = r;
        it.a1 = J;
        P.surv_list_items.push_back(it);
      }
    P.items = P.seed_items;
    // bound pass over LDS key tiles when tiles hold enough groups: one item per
    // (tile, 64-key-aligned share of its bounded range)
    // A bound workgroup takes 4/QW consecutive tiles of one sequence with the
    // same first bounded key, so its wavefronts hold 4 queries each; its key
    // range runs to the longest of their bounded ranges.
    if (P.tiled) {
      P.bound_gpw = 4 / P.QW;
      struct BlockInfo { int first, n, lo, hi; };
      std::vector<BlockInfo> blocks;
      for (size_t ti = 0; ti < tiles.size(); ++ti) {
        const TileInfo& t = tiles[ti];
        const GroupInfo& g = P.groups[t.first];
        const int lo = g.bound_lo, hi = g.bound_lo + g.n_bounded;
        if (!blocks.empty()) {
          BlockInfo& bk = blocks.back();
          const GroupInfo& h = P.groups[bk.first];
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
          P.bound_items.push_back(it);
        }
      }
      longest_first(P.bound_items, 0);
    }
    // probe: with enough tiles, the last tile (longest contexts) is seeded and
    // planned first; if its certificate can prune no query, the call scores
    // every tile densely with the dense path's items (regions 0..Jd-1)
    if (P.tiled && NT >= 8 && (cfg.flags & DOSA_NO_PROBE) == 0) {
      P.probe = true;
      const TileInfo& t = tiles.back();
      P.probe_group = t.first;
      P.probe_ngroups = t.n;
      P.probe_q0 = P.groups[t.first].q_row0;
      P.probe_nq = 0;
      for (int i = 0; i < t.n; ++i) P.probe_nq += P.groups[t.first + i].nq;
      // the probe tile's seed window in shares of at least 256 keys (up to 16
      // workgroups): on its own the tile would be scored by one workgroup
      const int wlo = std::max(0, t.n_last - P.W);
      const int f = std::min(P.F, wlo);
      P.Jp = (int)std::max<int64_t>(1, std::min<int64_t>(16, (t.n_last - wlo) / 256));
      for (int r = 0; r < P.Jp; ++r) {
        int lo, hi;
        range_split(wlo, t.n_last, r, P.Jp, 64, lo, hi);
        WorkItem it{};
        it.group = t.first;
        it.pad = t.n;
        it.region = r;
        it.a0 = 0; it.a1 = (r == 0) ? f : 0;
        it.b0 = lo; it.b1 = hi;
        P.probe_items.push_back(it);
      }
      P.Jd = dense_tiled_items(P.dense_items);
      P.R = std::max(P.R, std::max(P.Jd, P.Jp));
    }
    P.items.insert(P.items.end(), P.surv_tiled_items.begin(), P.surv_tiled_items.end());
    P.items.insert(P.items.end(), P.surv_list_items.begin(), P.surv_list_items.end());
    P.items.insert(P.items.end(), P.bound_items.begin(), P.bound_items.end());
    P.items.insert(P.items.end(), P.dense_items.begin(), P.dense_items.end());
    P.items.insert(P.items.end(), P.probe_items.begin(), P.probe_items.end());
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
  if (cfg.buffer_cap == 0) {
    int64_t max_n = 0;
    for (const auto& it : P.items) {
      int64_t n = (int64_t)(it.a1 - it.a0) + (it.b1 - it.b0);
      if (it.gather) {
        const int64_t nb = P.groups[it.group].n_bounded;
        n = std::max<int64_t>((nb + it.a1 - 1) / it.a1, std::min<int64_t>(nb, 2 * kUnionMinShare)) + 64;
      }
      max_n = std::max(max_n, n);
    }
    const double k = (double)topk;
    const double est = 1.3 * k * (1.0 + std::log(std::max((double)max_n, k) / k)) + 256.0;
    int64_t cap = std::min<int64_t>((int64_t)est, max_n + 64);
    cap = std::max<int64_t>(cap, topk + 64);
    P.cap = (int)((cap + 63) / 64 * 64);
  } else {
    P.cap = (cfg.buffer_cap + 63) / 64 * 64;
  }
  // workspace layout
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  P.o_groups = take(sizeof(GroupInfo) * std::max(G, 1));
  P.o_items = take(sizeof(WorkItem) * std::max<size_t>(P.items.size(), 1));
  if (!dense) P.o_seqinfo = take((size_t)(batch + 1) * sizeof(int32_t));   // copied with groups and items
  P.o_cand = take((size_t)P.total_q * P.R * P.cap * sizeof(u64));
  P.o_counts = take((size_t)P.total_q * P.R * sizeof(uint32_t));
  const int LS = 16 / P.QW;   // weighted-query terms per query
  P.o_lrows = take((size_t)P.total_q * LS * d * qbytes(q_dtype));
  P.o_lsig = take((size_t)P.total_q * LS * sizeof(float));
  P.o_lerr = take((size_t)P.total_q * 2 * sizeof(float));
  P.o_tshare = take((size_t)P.total_q * sizeof(uint32_t));
  if (!dense) {
    P.o_tau = take((size_t)P.total_q * sizeof(float));
    P.o_rows = take((size_t)P.total_q * 4 * d * qbytes(q_dtype));
    P.o_coef = take((size_t)P.total_q * 8 * sizeof(float));
    P.o_norms = take((size_t)std::max<int64_t>(P.total_k, 1) * sizeof(float));
    P.o_flag = take(sizeof(int32_t));
    P.o_masks = take((size_t)std::max(G, 1) * std::max(P.mask_words, 1) * sizeof(u64));
    P.o_lists = take((size_t)std::max<int64_t>(P.list_total, 1) * sizeof(int32_t));
    P.o_listlen = take((size_t)std::max(G, 1) * sizeof(int32_t));
    P.o_gflags = take((size_t)std::max(G, 1) * sizeof(int32_t));
    P.o_mode = take(sizeof(int32_t));
    P.o_order = take(sizeof(int32_t) * std::max<size_t>(P.surv_tiled_items.size(), 1));
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
    const size_t end = dense ? P.o_items + n_items : P.o_seqinfo + (size_t)(batch + 1) * sizeof(int32_t);
    std::vector<char> stage(end - P.o_groups, 0);
    std::memcpy(stage.data(), P.groups.data(), sizeof(GroupInfo) * P.groups.size());
    std::memcpy(stage.data() + (P.o_items - P.o_groups), P.items.data(), n_items);
    if (!dense) {
      int32_t* cu = reinterpret_cast<int32_t*>(stage.data() + (P.o_seqinfo - P.o_groups));
      cu[0] = 0;
      for (int b = 0; b < batch; ++b) cu[b + 1] = cu[b] + kv_lens[b];
    }
    e = hipMemcpyAsync(ws + P.o_groups, stage.data(), stage.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(plan)");
  }
  if (st) {
    unsigned long long add[11] = {P.pairs_total, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    e = launch_stats_add(st, add, stream);
    if (e != hipSuccess) return fail_hip(e, "stats");
  }
  Inputs in{q, q_scale, w, k, k_scale, page_table, page_size, max_pages};
  PrepLaunch pr{q, w, P.total_q, ws + P.o_lrows, reinterpret_cast<float*>(ws + P.o_lsig),
                reinterpret_cast<float*>(ws + P.o_lerr), dense ? nullptr : reinterpret_cast<int32_t*>(ws + P.o_flag),
                reinterpret_cast<uint32_t*>(ws + P.o_tshare)};
  uint32_t* tshare = kShareTheta ? reinterpret_cast<uint32_t*>(ws + P.o_tshare) : nullptr;
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
    sl.tiled = P.tiled ? 1 : 0;
    sl.role = ROLE_DENSE;
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
    const size_t off_surv = P.seed_items.size(), off_list = off_surv + P.surv_tiled_items.size(),
                 off_bound = off_list + P.surv_list_items.size(), off_dense = off_bound + P.bound_items.size(),
                 off_probe = off_dense + P.dense_items.size();
    int32_t* mode = P.probe ? reinterpret_cast<int32_t*>(ws + P.o_mode) : nullptr;
    // 1b. probe: seed pass, threshold and plan of the last tile only, then the
    //     decision whether the call runs the certificate pipeline or dense scoring
    if (P.probe) {
      PassScope ps(P_PROBE, stream);
      ScoreLaunch pb{};
      pb.theta_share = tshare;
      pb.in = in;
      pb.lrows = pr.rows;
      pb.lsig = pr.sig;
      pb.groups = dg;
      pb.items = di + off_probe;
      pb.n_items = P.Jp;
      pb.cb = cb;
      pb.topk = topk;
      pb.scored_slot = 1;
      pb.tiled = 1;
      pb.role = ROLE_SEED;
      e = launch_score(P.combo, H, d, pb, stream);
      if (e != hipSuccess) return fail_hip(e, "probe seed kernel launch");
      SelectLaunch pt{};
      pt.cb = cb;
      pt.q_first = P.probe_q0;
      pt.total_q = P.probe_nq;
      pt.topk = topk;
      pt.r0 = 0;
      pt.r1 = P.Jp;
      pt.tau_out = tau;
      e = launch_select_tau(pt, stream);
      if (e != hipSuccess) return fail_hip(e, "probe select kernel launch");
      PlanLaunch pp{};
      pp.in = in;
      pp.groups = dg + P.probe_group;
      pp.n_groups = P.probe_ngroups;
      pp.num_proxies = cfg.num_proxies;
      pp.seed_window = P.W;
      pp.neg_frac = cfg.neg_support_frac;
      pp.flags = cfg.flags;
      pp.tau = tau;
      pp.lerr = pr.err;
      pp.prunes = prunes;
      pp.rows = ws + P.o_rows;
      pp.coef = coef;
      e = launch_plan(P.combo, H, d, pp, stream);
      if (e != hipSuccess) return fail_hip(e, "probe plan kernel launch");
      e = launch_probe_decide(coef, P.probe_q0, P.probe_nq, mode, st, stream);
      if (e != hipSuccess) return fail_hip(e, "probe decision kernel launch");
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
    sl.tiled = 1;
    sl.role = ROLE_SEED;
    {
      PassScope ps(P_SCORE_SEED, stream);
      e = launch_score(P.combo, H, d, sl, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "seed score kernel launch");
    // 3. tau = K-th largest seed score
    SelectLaunch ts{};
    ts.mode = mode;
    ts.run_if = MODE_PRUNED;
    ts.cb = cb;
    ts.total_q = (int32_t)P.total_q;
    ts.topk = topk;
    ts.r0 = 0;
    ts.r1 = P.Js;
    ts.tau_out = tau;
    {
      PassScope ps(P_SELECT_SEED, stream);
      e = launch_select(ts, stream);
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
      PassScope ps(P_PLAN, stream);
      e = launch_plan(P.combo, H, d, pl, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "plan kernel launch");
    // 4b. per-key norms for the bound pass; the launch returns at once when the
    //     plan found no query whose certificate can prune
    NormLaunch nl{in, cu_dev, batch, P.total_k, max_kv, norms, cfg.debug_ub != nullptr ? nullptr : prunes};
    {
      PassScope ps(P_NORMS, stream);
      e = launch_key_norms(P.combo, d, nl, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "key norm kernel launch");
    // 5. bound pass -> survivor bitmasks
    BoundLaunch bl{};
    bl.mode = mode;
    bl.run_if = MODE_PRUNED;
    bl.in = in;
    bl.groups = dg;
    bl.n_groups = G;
    bl.rows = ws + P.o_rows;
    bl.coef = coef;
    bl.norms = norms;
    bl.masks = masks;
    bl.mask_words = std::max(P.mask_words, 1);
    bl.debug_ub = cfg.debug_ub;
    bl.debug_ld = max_kv;
    bl.splits = P.bound_splits;
    if (!P.bound_items.empty()) {
      bl.items = di + off_bound;
      bl.n_items = (int)P.bound_items.size();
      bl.groups_per_wave = P.bound_gpw;
    }
    bl.stats = st;
    {
      PassScope ps(P_BOUND, stream);
      e = launch_bound(P.combo, H, d, bl, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "bound kernel launch");
    // 6. compaction -> survivor key lists
    CompactLaunch cl{};
    cl.groups = dg;
    cl.tiles = di;                    // the seed items: Js per tile, the first names the tile
    cl.tile_stride = P.Js;
    cl.n_tiles = P.Js > 0 ? (int)P.seed_items.size() / P.Js : 0;
    cl.allow_union = P.tiled ? 1 : 0;
    cl.coef = coef;
    cl.masks = masks;
    cl.mask_words = std::max(P.mask_words, 1);
    cl.lists = lists;
    cl.list_len = list_len;
    cl.group_flags = gflags;
    cl.cb = cb;
    cl.r0 = P.Js;
    cl.r1 = P.Js + P.J;
    cl.mode = mode;
    cl.run_if = MODE_PRUNED;
    {
      PassScope ps(P_COMPACT, stream);
      e = launch_compact(cl, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "compact kernel launch");
    // 7. survivors scored with all heads into regions Js..Js+J-1, threshold starts at tau:
    //    flagged tiles take the tiled kernel over their union list (or, in calls
    //    without tiles, over the bounded range), the other groups walk their own lists
    ScoreLaunch ml{};
    ml.theta_share = tshare;
    ml.mode = mode;
    ml.run_if = MODE_PRUNED;
    ml.in = in;
    ml.lrows = pr.rows;
    ml.lsig = pr.sig;
    ml.groups = dg;
    ml.cb = cb;
    ml.theta_init = tau;
    ml.lists = lists;
    ml.list_len = list_len;
    ml.topk = topk;
    ml.stats = st;
    ml.scored_slot = 4;
    ml.tile_flags = gflags;
    ml.role = ROLE_SURVIVORS;
    {
      PassScope ps(P_SURV_TILES, stream);
      ml.items = di + off_surv;
      ml.n_items = (int)P.surv_tiled_items.size();
      ml.tiled = P.tiled ? 1 : 0;
      ml.flag_mode = 1;
      // union shares are cut on the device: launch them longest first
      if (P.tiled && ml.n_items > 0 && ml.n_items <= kMaxOrderItems) {
        OrderLaunch ol{ml.items, ml.n_items, list_len, gflags, reinterpret_cast<int32_t*>(ws + P.o_order), mode,
                       MODE_PRUNED};
        e = launch_order(ol, stream);
        ml.order = ol.order;
      }
      if (e == hipSuccess) e = launch_score(P.combo, H, d, ml, stream);
    }
    if (e == hipSuccess) {
      PassScope ps(P_SURV_LISTS, stream);
      ml.items = di + off_list;
      ml.n_items = (int)P.surv_list_items.size();
      ml.tiled = 0;
      ml.flag_mode = 2;
      ml.scored_slot2 = 8;
      e = launch_score(P.combo, H, d, ml, stream);
    }
    if (e != hipSuccess) return fail_hip(e, "survivor score kernel launch");
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
      dl.tiled = 1;
      dl.role = ROLE_DENSE;
      PassScope ps(P_SCORE_DENSE, stream);
      e = launch_score(P.combo, H, d, dl, stream);
      if (e != hipSuccess) return fail_hip(e, "dense score kernel launch");
    }
  }
  SelectLaunch se{};
  se.cb = cb;
  se.total_q = (int32_t)P.total_q;
  se.topk = topk;
  se.r0 = 0;
  se.r1 = dense ? P.R : P.Js + P.J;   // pruned path: seed then survivor regions
  se.out_idx = out_idx;
  se.out_score = out_score;
  se.tau_out = nullptr;
  se.r1_unpruned = P.probe ? P.Jd : P.R;
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

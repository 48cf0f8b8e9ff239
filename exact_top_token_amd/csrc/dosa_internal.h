// Internal declarations shared by the host planner and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dosa_indexer.h"

namespace dosa {

// Operand combinations the kernels are built for.
enum Combo : int { C_F32 = 0, C_BF16 = 1, C_FP8 = 2, C_BF16Q_FP8K = 3 };

// Which pass a scoring launch belongs to (selects a kernel of its own name).
enum Role : int { ROLE_DENSE = 0, ROLE_SEED = 1, ROLE_SURVIVORS = 2 };

// How a pruned-path call proceeds once its probe tile has been planned: the
// certificate pipeline, or dense scoring of every key when the certificate
// cannot prune any query of the probe tile.  Launches carry a mode pointer
// and the mode they run in; the others return at once.
enum DosaMode : int { MODE_PRUNED = 0, MODE_UNPRUNED = 1 };

__device__ __forceinline__ bool skip_launch(const int32_t* mode, int32_t run_if) {
  return mode != nullptr && run_if >= 0 && *mode != run_if;
}

constexpr int kTileWaves = 8;   // wavefronts (query groups) per tiled scoring workgroup
// A tile's union survivor list is scored in up to WorkItem::a1 shares of at
// least this many keys each (shorter lists take fewer workgroups).
constexpr int kUnionMinShare = 1024;

// A query group: up to 4 consecutive queries of one sequence, scored together
// by one wavefront (MFMA rows = group queries x head slots).
struct GroupInfo {
  int64_t list_off;  // start of the group's survivor list (DoSA); the lists of a call can
                     // hold more than 2^31 entries (long contexts x many query groups)
  int32_t seq;       // sequence index
  int32_t q_row0;    // global row of the first query
  int32_t nq;        // queries in the group
  int32_t pos0;      // position of the first query (queries are consecutive)
  int32_t key_base;  // contiguous storage: row of the sequence's key 0
  int32_t list_cap;  // capacity of that list
  int32_t n_bounded; // keys the bound pass covers: [bound_lo, bound_lo + n_bounded)
  int32_t bound_lo;  // first bounded key (end of the seed prefix)
  int32_t norm_base; // index of the sequence's key 0 in the per-key norm array
  int32_t tile_first;// first group of the tile (<= 8 consecutive groups) this group belongs to
  int32_t tile_n;    // groups in that tile
  int32_t blk_base;  // index of the sequence's first 64-key block in the key-block summaries
};

// A share of scoring: a group (list kernel) or a tile of up to 8 groups
// starting at `group` (tiled kernel, `pad` = groups in the tile), a candidate
// region and the keys.  Range mode walks [a0,a1) then [b0,b1), each from the
// top down; gather mode walks split a0 of a1 of the group's survivor list.
struct WorkItem {
  int32_t group;
  int32_t region;
  int32_t a0, a1;
  int32_t b0, b1;
  int32_t gather;
  int32_t pad;
  int32_t nparts;   // split thresholds: the launch's disjoint sweeps over this item's queries' keys
                    // (the items of its tile or group in the launch), 0 = not counted
};

// Head slots the kernels are built for: the head count rounded up to 8, 16,
// 32 or 64.  Slots past the real count hold zero queries with zero weight, so
// they add nothing to a score and are neither positive nor negative heads.
__host__ __device__ constexpr int padded_heads(int H) {
  return H <= 8 ? 8 : (H <= 16 ? 16 : (H <= 32 ? 32 : 64));
}

// Where the inputs live, as the kernels see them.
struct Inputs {
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
  const int32_t* page_table;  // NULL = contiguous
  int32_t page_size;
  int32_t max_pages;
  int32_t H;                  // heads per query: the row stride of q and w (<= the kernel's head slots)
  int32_t page_shift;         // log2(page_size) when it is a power of two, else -1
};

// Candidate buffers, region-major: entry (q_row, region, i) at
// cand[(region*rows + q_row)*cap + i], count at counts[region*rows + q_row].
// The rows of one region are contiguous, so a scoring launch that fills a few
// regions writes a compact span of memory however many regions the call has.
struct CandBuf {
  unsigned long long* cand;
  uint32_t* counts;
  int32_t R;
  int32_t cap;
  int64_t rows;              // query rows the buffer holds
  int64_t q_base;            // global row of its first query (0: the whole call)
  __host__ __device__ unsigned long long* row(int64_t q, int r) const {
    return cand + ((int64_t)r * rows + (q - q_base)) * cap;
  }
  __host__ __device__ uint32_t* count(int64_t q, int r) const { return counts + (int64_t)r * rows + (q - q_base); }
};

// Weighted query sums (see prep.hip): rows [total_q, 16/QW, d] in the query
// operand type, sig [total_q, 16/QW] term scales, err [total_q, 2] =
// (||qbar - represented qbar||, sum_j sigma_j ||f_j||), unscaled units.
struct PrepLaunch {
  const void* q;
  const float* w;
  int32_t H;            // heads per query (row stride of q and w)
  int64_t total_q;
  void* rows;
  float* sig;
  float* err;
  int32_t* flag;        // [2] cleared here (query 0): the plan's "some query can prune" flag and the
                        // probe plan's ticket counter, or NULL
  uint32_t* tshare;     // [total_q] cleared here: the shared running thresholds (ScoreLaunch)
  uint32_t* tpart;      // [total_q, n_parts] cleared here: the split thresholds (ScoreLaunch), or NULL
  int32_t n_parts;
  uint32_t* counts;     // candidate counts [n_regions, total_q], cleared here: a region no item
  int32_t n_regions;    // of the call fills reads as empty in the final merge
};

struct ScoreLaunch {
  Inputs in;
  const void* lrows;         // weighted-query rows (PrepLaunch::rows)
  const float* lsig;         // their scales (PrepLaunch::sig)
  const GroupInfo* groups;
  const WorkItem* items;
  int32_t n_items;
  CandBuf cb;
  const float* theta_init;   // [total_q] or NULL (-inf)
  uint32_t* theta_share;     // [total_q] order-preserving images of running thresholds that every
                             // launch of the call publishes to and adopts from (0 = none yet), or NULL
  // Split thresholds: the launch scores each query's keys in P = nparts
  // disjoint sweeps (its items; every one present).  Sweep r publishes the
  // image of its ceil(K / P)-th largest score so far in
  // theta_part[q * part_stride + part_base + r]; once all P are published,
  // their minimum has at least K scores at or above it over the sweeps
  // together, a valid threshold for each of them.  NULL: off.
  uint32_t* theta_part;
  int32_t part_stride, part_base;
  int32_t part_rbase;        // region of sweep 0: sweep index = item region - part_rbase; the sweep
                             // count is the item's nparts
  const int32_t* lists;      // survivor lists (gather mode)
  const int32_t* list_len;   // survivor list length per group (gather mode)
  const int32_t* list_start; // per group: start of its list after GroupInfo::list_off (or NULL: 0)
  int64_t list_stride;       // > 0: group g's list starts at lists + g * list_stride instead
  int32_t topk;
  int32_t scored_slot;       // dosa_stats field (u64 index) that counts scored pairs
  int32_t scored_slot2;      // a second field that counts them too (0 = none)
  int32_t tiled;             // 1: score_tiled_kernel, 0: score_list_kernel, 2: score_split_kernel
                             // (regions r * kTileWaves + wavefront of the items' regions r)
  const int32_t* tile_flags; // per group: 1 if the certificate prunes nothing in its tile (or NULL)
  const int32_t* order;      // [n_items]: workgroup b takes item order[b] (longest first), or NULL
  int32_t flag_mode;         // 0: run every item; 1: only tiles flagged; 2: only groups whose tile is not
  int32_t role;              // Role
  unsigned long long* stats; // dosa_stats as u64[12] or NULL
  const int32_t* mode;       // NULL: always run; else run only if *mode == run_if (see DosaMode)
  int32_t run_if;
};

struct SelectLaunch {
  CandBuf cb;
  int32_t total_q;
  int32_t topk;
  int32_t r0, r1;            // regions merged: [r0, r1)
  int32_t* out_idx;          // NULL: threshold-only mode
  float* out_score;
  float* tau_out;            // K-th score per query (-inf if fewer than K), or NULL
  float* tau_copy;           // a second copy of tau_out (the caller's debug array), or NULL
  float* coef_tau;           // plan coefficients whose threshold slot (coef[5]) takes tau too, or NULL
  int32_t sorted;
  unsigned long long* stats;
  int32_t q_first;           // rows q_first .. q_first + total_q - 1
  int32_t r1_unpruned;       // regions merged instead of [r0, r1) when *mode == MODE_UNPRUNED
  const int32_t* mode;       // NULL: always run; else run only if *mode == run_if (see DosaMode)
  int32_t run_if;
};

// Certificate plan: per query 4 operand rows of d elements in the query
// storage type (proxy rows first, then terms of the negative aggregate) and
// kCoefStride fp32 coefficients:
//   coef[0..3] : per-row multiplier (proxy rows: c_p * q_scale; aggregate
//                rows: sigma_j * q_scale)
//   coef[4]    : rho' * q_scale (joint residual constant plus rounding margin)
//   coef[5]    : tau (seed threshold)
//   coef[6]    : number of proxy rows p (rows p..3 are aggregate terms)
//   coef[7]    : 1 if the certificate cannot prune any key of this query
//   coef[8..11]: Euclidean norm of each row's stored values (rounded up), for
//                the key-block bound
constexpr int kCoefStride = 16;
struct PlanLaunch {
  Inputs in;
  const GroupInfo* groups;
  int32_t n_groups;
  int32_t num_proxies;
  int32_t seed_window;
  float neg_frac;
  uint32_t flags;
  const float* tau;          // [total_q], or NULL in a probe plan (estimated threshold, below)
  const float* lerr;         // [total_q, 2] weighted-query representation error and magnitude
  void* rows;                // [total_q, 4, d] query storage type
  float* coef;               // [total_q, 8]
  int32_t* prunes;           // set to 1 when some query's certificate can prune (or NULL)
  const int32_t* mode;       // NULL: always run; else run only if *mode == run_if (see DosaMode)
  int32_t run_if;
  // probe decision (or NULL): the last of the decide_nq planned queries (a
  // ticket counter, zeroed by the prep kernel) sets *decide_mode from the
  // prunes flag their plans raised (prunes must be set)
  int32_t* ticket;
  int32_t decide_nq;
  int32_t* decide_mode;
  unsigned long long* stats;
  // probe plans (tau == NULL): the threshold is estimated from the sampled
  // window keys instead of read, as the sample's quantile at topk over the
  // query's seed keys (the first seed_prefix keys and its window); a cost
  // decision only, the certificate pipeline plans every query again
  int32_t topk;
  int32_t seed_prefix;
};

struct BoundLaunch {
  Inputs in;
  const GroupInfo* groups;
  int32_t n_groups;
  const void* rows;
  const float* coef;
  const float* norms;        // per logical key, sequences back to back
  unsigned long long* masks; // [n_groups, mask_words]
  int32_t mask_words;
  float* debug_ub;           // [total_q, debug_ld] or NULL
  int32_t debug_ld;
  unsigned long long* debug_mask;  // [total_q, debug_mask_ld] survivor bits per (query, key) or NULL
  int32_t debug_mask_ld;
  const uint8_t* blk_code;   // key-block centres [blocks, d] in the key storage type, or NULL (no block test)
  const float* blk_info;     // [blocks, 4]: centre scale, radius, largest key norm, centre norm
  int32_t splits;            // key splits per group (grid = n_groups * splits; per-group kernel)
  const WorkItem* items;     // tiled kernel: one per (query block, key share): group = first group,
                             // pad = groups, [a0, a1) keys, b0 = share index; NULL = per-group kernel
  int32_t n_items;
  int32_t groups_per_wave;   // tiled kernel: 4 / (queries per group)
  int32_t count_skipped;     // 1: skipped groups are counted (stats slot 7); 0 in a call's second round
  unsigned long long* stats;
  const int32_t* mode;       // NULL: always run; else run only if *mode == run_if (see DosaMode)
  int32_t run_if;
};

struct CompactLaunch {
  const GroupInfo* groups;
  const WorkItem* tiles;     // tile i's first group is tiles[i * tile_stride].group
  int32_t tile_stride;
  int32_t n_tiles;           // grid: one workgroup per tile
  int32_t allow_union;       // 1: tiles may be routed to the tiled kernel's union lists
  int32_t force_lists;       // 1 (with allow_union): every tile's groups get their own lists
  const float* coef;         // plan coefficients (coef[7]: hopeless flag per query)
  const unsigned long long* masks;
  int32_t mask_words;
  int32_t* lists;
  int32_t* list_len;
  int32_t* list_start;       // out: per group, start of its list after list_off (the groups of a tile
                             // with query tiles share one list area: a union list, or their own
                             // lists packed one after the other)
  int32_t* group_flags;      // out: 1 if the group's tile is scored whole: over its union list
                             // (allow_union) or over its bounded range
  CandBuf cb;                // candidate counts of regions [r0, r1) of the tile's queries are
  int32_t r0, r1;            // zeroed here (the survivor pass writes only the regions it fills,
                             // the final merge reads them all)
  const int32_t* mode;       // NULL: always run; else run only if *mode == run_if (see DosaMode)
  int32_t run_if;
};

// Launch order of the tiled survivor pass: its items (share r of a tile's
// union list) sorted by share length, longest first, so that the launch's
// tail holds the short shares.  One workgroup; at most kMaxOrderItems items.
constexpr int kMaxOrderItems = 4096;
struct OrderLaunch {
  const WorkItem* items;
  int32_t n_items;
  const int32_t* list_len;
  const int32_t* tile_flags;
  int32_t* order;            // out: [n_items]
  const int32_t* mode;
  int32_t run_if;
};

struct NormLaunch {
  Inputs in;
  const int32_t* cu_kv;      // [batch+1] logical key offsets
  int32_t batch;
  int64_t total_k;
  int32_t max_kv;            // longest sequence
  float* norms;              // [total_k]
  const int32_t* needed;     // NULL, or the plan's flag: 0 = no query can prune, nothing to do
  const int32_t* cu_blk;     // [batch+1] offsets of the sequences' 64-key blocks (key-block kernel)
  uint8_t* blk_code;         // [blocks, d] centres in the key storage type (key-block kernel)
  float* blk_info;           // [blocks, 4] (key-block kernel)
};

// Extra seed keys (dosa_config::seed_idx): per query group, the union of its
// queries' rows restricted to the group's bounded keys, sorted and without
// repeats, at lists + group * stride; its length in list_len[group].
constexpr int kMaxSeedCount = 4096;          // entries per query row
constexpr int kSeedUnionMax = 4 * kMaxSeedCount;   // entries of a group's rows (<= 4 queries)
struct SeedUnionLaunch {
  const GroupInfo* groups;
  int32_t n_groups;
  const int32_t* seed_idx;   // [total_q, seed_count]
  int32_t seed_count;
  int32_t* lists;            // out: [n_groups, stride]
  int64_t stride;
  int32_t* list_len;         // out: [n_groups]
  const int32_t* mode;       // NULL: always run; else run only if *mode == run_if (see DosaMode)
  int32_t run_if;
};

constexpr int kKeyBlock = 64;       // keys per key block (= the bound pass's key tile)
constexpr int kMaxBoundTiles = 4096;// key tiles of a bound item that the block test covers

// Launchers (return hipError_t of the launch).
hipError_t launch_score(int combo, int H, int d, const ScoreLaunch& p, hipStream_t s);
hipError_t launch_prep(int combo, int H, int d, const PrepLaunch& p, hipStream_t s);
hipError_t launch_select(const SelectLaunch& p, hipStream_t s);
hipError_t launch_key_norms(int combo, int d, const NormLaunch& p, hipStream_t s);
hipError_t launch_key_blocks(int combo, int d, const NormLaunch& p, hipStream_t s);
hipError_t launch_plan(int combo, int H, int d, const PlanLaunch& p, hipStream_t s);
hipError_t launch_bound(int combo, int H, int d, const BoundLaunch& p, hipStream_t s);
hipError_t launch_compact(const CompactLaunch& p, hipStream_t s);
hipError_t launch_order(const OrderLaunch& p, hipStream_t s);
hipError_t launch_seed_union(const SeedUnionLaunch& p, hipStream_t s);
hipError_t launch_stats_add(unsigned long long* stats, const unsigned long long* host_vals, hipStream_t s);

bool combo_supported(int combo, int H, int d);
int tile_waves();

}  // namespace dosa

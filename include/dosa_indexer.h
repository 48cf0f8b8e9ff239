/*
 * dosa_indexer.h -- exact Top-K selection for the DSA sparse-attention indexer
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (DoSA pages: podcast transcript of "DOSA: Dots Sparse
 * Attention", Method section, problem formulation; the DSA indexer score):
 * every query t carries H indexer heads with query vectors q[t,h,:] and
 * signed weights w[t,h]; all heads share one key k[s,:] per token.  The score
 * of key s for query t is
 *
 *     S(t,s) = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])
 *
 * and each query keeps the K visible keys of highest score.  Causality: query
 * i of sequence b sits at position kv_lens[b] - q_lens[b] + i and sees the
 * keys at positions 0..position.  Ties are broken towards the lower position.
 * When fewer than K keys are visible, all of them are returned followed by -1.
 *
 * Two entry points compute the same set:
 *   dsa_indexer_topk   scores every visible key (dense scoring with a
 *                      streaming Top-K; the plain method).
 *   dosa_indexer_topk  the DoSA way (same pages, Method section: seed subset
 *                      threshold, certificate built from nonnegative head
 *                      projections, a joint residual bound and an
 *                      activation-informed negative-head aggregate; zicq.com
 *                      summary, items 1-3; picx.dev item, sections 02-03):
 *                      a seed pass scores a seed subset exactly and takes its
 *                      K-th score as a threshold tau; a bound pass computes a
 *                      conservative upper bound per key; keys whose bound is
 *                      below tau are dropped; survivors are compacted and
 *                      scored with all heads; then the exact Top-K.  The
 *                      selected set is identical to dsa_indexer_topk's, bit
 *                      for bit, for every configuration.
 *
 * Layouts (all row-major, all pointers below are DEVICE pointers unless said):
 *   q        [total_q, H, d] of q_dtype; queries of the batch back to back
 *            (total_q = sum q_lens).
 *   q_scale  [total_q] fp32, required iff q_dtype == DOSA_FP8_E4M3FN (one
 *            scale per query token across all heads); ignored otherwise.
 *   w        [total_q, H] fp32 (any sign).
 *   k        contiguous (page_table == NULL): [total_k, d] of k_dtype,
 *            sequence b's keys at rows sum(kv_lens[0..b-1]) + position;
 *            paged: [num_pages, page_size, d], logical key j of sequence b in
 *            pool page page_table[b*max_pages + j/page_size], slot j%page_size.
 *   k_scale  per key token fp32 ([total_k] or [num_pages, page_size]),
 *            required iff k_dtype == DOSA_FP8_E4M3FN.
 *   fp8 values are OCP E4M3FN; the value of a code is scale * decode(code).
 *   q_lens, kv_lens  HOST int32 [batch], 0 <= q_lens[b] <= kv_lens[b].
 *   out_idx  [total_q, topk] int32: logical key positions, -1 padding.
 *   out_score [total_q, topk] fp32 or NULL: the fp32 score of each returned
 *            key (-inf padding).
 *   Row order inside out_idx is unspecified unless DOSA_SORTED is set (then
 *   score descending, position ascending); it is deterministic run to run.
 *
 * Supported: d in {64, 128}; H a multiple of 8 in [8, 64]; 1 <= topk <= 4096;
 * (q_dtype, k_dtype) in {(F32,F32), (BF16,BF16), (FP8,FP8), (BF16,FP8)};
 * contiguous keys: sum(kv_lens) < 2^31 and kv_lens[b] * d * sizeof(k) < 2^32;
 * sum(q_lens) < 2^31.  Other shapes return DOSA_ERR_UNSUPPORTED.
 * Inputs must be finite.
 *
 * Ownership and synchronisation: the caller owns every buffer, including the
 * workspace (size from dosa_workspace_size).  The library allocates no device
 * memory and keeps no data between calls; everything is ordered on `stream`
 * (a hipStream_t, NULL = default stream) and no call waits for the device.
 * A pruned call with query tiles that runs the probe (see DOSA_NO_PROBE),
 * has at least 2^26 causal pairs and whose dense alternative fits in two
 * workgroups per CU forks the certificate stages onto
 * a side stream the library creates once per device (default priority, kept
 * until the process ends) and joins it back into `stream` before its final
 * selection, so `stream` order covers the whole call (graph capture too).
 * Outputs, workspace contents and stats are valid once the stream has
 * completed.  Calls on distinct workspaces/streams may run concurrently;
 * their certificate stages then share the device's side stream.
 *
 * Errors: 0 on success or a negative dosa_status.  On error nothing has been
 * enqueued.  No C++ exception crosses this interface.
 */
#ifndef DOSA_INDEXER_H_
#define DOSA_INDEXER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DOSA_F32 = 0,
  DOSA_BF16 = 1,
  DOSA_FP8_E4M3FN = 2
} dosa_dtype;

typedef enum {
  DOSA_OK = 0,
  DOSA_ERR_INVALID_ARG = -1,     /* null pointer, bad length, q_lens > kv_lens, ... */
  DOSA_ERR_UNSUPPORTED = -2,     /* dtype combination, d, H or topk outside the supported set */
  DOSA_ERR_WORKSPACE = -3,       /* workspace NULL or smaller than dosa_workspace_size */
  DOSA_ERR_HIP = -4              /* a HIP runtime call or kernel launch failed */
} dosa_status;

/* flags */
#define DOSA_NO_PRUNE 0x1u        /* dosa_indexer_topk: skip the bound pass (every key survives) */
#define DOSA_SORTED 0x2u          /* rows of out_idx in (score desc, position asc) order */
#define DOSA_SEPARABLE_RHO 0x4u   /* residual bound sum_h w_h ||r_h|| instead of the joint bound */
#define DOSA_NO_NEGATIVE 0x8u     /* drop the negative-head aggregate from the bound */
#define DOSA_KEY_BLOCKS 0x20u     /* dosa_indexer_topk: key-block test in the bound pass (calls with query
                                     tiles): per 64-key block a centre, radius and largest norm give one
                                     bound for all its keys (certificates over key blocks, the DoSA
                                     transcript's Conclusion); a block below tau for every query of a
                                     32-query bound tile is never loaded.  Off by default: on the
                                     correlated 128K recipe it skips 5.6% of the tiles and the test
                                     costs more than that saves */
#define DOSA_NO_PROBE 0x10u       /* dosa_indexer_topk: no probe, always the certificate pipeline
                                     (by default a call with >= 8 query tiles first plans its last
                                     tile -- a decode-like call with >= 8 sequences its groups, up
                                     to 256 of them --
                                     with the threshold estimated from the plan's sampled seed-window
                                     keys and, if the certificate prunes no query there, scores every
                                     key densely; the result is the same either way) */
#define DOSA_TWO_ROUNDS 0x40u     /* dosa_indexer_topk, calls with query tiles: the threshold is
                                     refined once within the call (the DoSA transcript, Method: the
                                     stages repeat over tiles of keys as the standings refine).
                                     Round 1 bounds and scores the newer half of each tile's bounded
                                     keys against the seed threshold; the K-th largest exact score
                                     of the seed and round-1 candidates (a valid lower bound of the
                                     K-th score: K distinct keys reach it) becomes the threshold of
                                     round 2 over the older half.  debug_tau keeps round 1's
                                     threshold; debug_mask bits of round-2 keys are against the
                                     raised one */
#define DOSA_GROUP_LISTS 0x80u    /* dosa_indexer_topk, calls with query tiles: every tile's survivors
                                     go to the per-group streams (each query group's own compacted
                                     list, scored one wavefront per group; a group holds the queries
                                     one wavefront scores together: 4 for fp8, 2 for bf16, 1 for
                                     fp32 at H = 64, d = 128) instead of the shared stream (the
                                     tile's union list, whose keys serve all its queries), the two
                                     kinds of survivor stream of the DoSA transcript (Method: GPU
                                     kernel design).  By default compaction picks the union unless
                                     it is 8x the groups' lists together.  The result is the same
                                     either way; the workspace reserves one list of every bounded
                                     key per group */

/* Knobs of dosa_indexer_topk.  None of them changes the selected set; they
 * only change how much work the certificate saves. */
typedef struct {
  int32_t num_proxies;      /* positive heads evaluated exactly in the bound: 0..3 (default 3;
                               the bound kernels give each query 4 MFMA rows: p proxy rows and
                               4 - p rows for the negative-head aggregate) */
  int32_t seed_window;      /* seed = the last seed_window visible keys ... (default 4*topk, >= 64) */
  int32_t seed_prefix;      /* ... plus the first seed_prefix keys (default 64) */
  int32_t buffer_cap;       /* entries per candidate region (each query has one region per key
                               range scored in parallel); 0 = automatic (default): about
                               1.3*topk*(1 + ln(range/topk)) + 256 for the longest range, so
                               that regions rarely overflow; else >= topk + 64 */
  int32_t key_splits;       /* key ranges scored in parallel per query group; 0 = automatic */
  float neg_support_frac;   /* negative head joins the aggregate if positive on >= this
                               fraction of the sampled seed keys (default 0.5) */
  uint32_t flags;           /* DOSA_* flags */
  float* debug_ub;          /* optional DEVICE [total_q, max_kv] fp32: certificate value per
                               bounded key (untouched elsewhere); for testing only */
  float* debug_tau;         /* optional DEVICE [total_q] fp32: each query's seed threshold tau
                               (the K-th largest exactly scored seed score, -inf with fewer than
                               K seeds); written only when the call runs the certificate
                               pipeline (always with DOSA_NO_PROBE); for testing only */
  uint64_t* debug_mask;     /* optional DEVICE [total_q, ceil(max_kv/64)] u64, zeroed by the
                               caller: bit s%64 of word s/64 is OR-ed in for every bounded key s
                               whose certificate reached tau for that query (every bounded key
                               of a query whose plan found nothing to prune); seed keys are not
                               marked; for testing only */
  const int32_t* seed_idx;  /* optional DEVICE [total_q, seed_count] int32: extra seed keys per query,
                               scored exactly and used for tau only -- e.g. the previous decode
                               step's Top-K (the DoSA transcript, Experiments: decode reuses the
                               scores of recently selected keys) or a candidate set shared by a
                               group of nearby queries (the PIVOT record: one scan per query
                               group).  Logical key positions; entries outside the keys that get
                               a certificate (negative, past the query, or inside the seed prefix
                               or window) and repeats are ignored, -1 may pad a row.  Queries
                               scored together (up to 4 consecutive queries of a sequence) share
                               the union of their rows, which keeps every seed visible to each of
                               them.  Any content leaves the selected set unchanged; keys that
                               score high raise tau and so the pruning */
  int32_t seed_count;       /* entries per row of seed_idx, 0..4096 (0 = none, the default) */
  int32_t reserved;         /* set to 0 */
} dosa_config;

/* Device-resident counters, accumulated (not reset) by each call that gets a
 * non-NULL pointer.  Pairs are causal (query, visible key) pairs. */
typedef struct {
  uint64_t pairs_total;        /* all visible pairs */
  uint64_t pairs_seed;         /* pairs scored exactly in the seed pass */
  uint64_t pairs_bounded;      /* pairs given a certificate (non-seed) */
  uint64_t pairs_survived;     /* bounded pairs whose certificate reached tau */
  uint64_t pairs_scored;       /* pairs scored with all heads after the seed (incl. tile union) */
  uint64_t candidates_written; /* entries appended to candidate buffers */
  uint64_t reselects;          /* in-kernel buffer re-selections */
  uint64_t groups_skipped;     /* query groups whose certificate could prune nothing */
  uint64_t pairs_scored_list;  /* the part of pairs_scored scored from compacted survivor lists */
  uint64_t keys_streamed;      /* key rows the bound pass read (once per query tile or group that
                                  streamed them; skipped groups read none) */
  uint64_t calls_unpruned;     /* dosa_indexer_topk calls scored densely: the certificate could
                                  prune no query the probe planned (the call's last query tile, or
                                  every group of a decode-like call) */
  uint64_t key_blocks_skipped; /* 64-key tiles the bound pass never loaded: the key-block bound
                                  (centre, radius and largest norm of the block's keys) was below
                                  tau for every query of the query tile that needed them */
} dosa_stats;

/* Fill *cfg with the defaults for a given topk. */
int dosa_default_config(int32_t topk, dosa_config* cfg);

/* Bytes of device workspace the call with these shapes needs. q_lens/kv_lens
 * are HOST arrays.  paged != 0 if a page table will be passed.  cfg NULL =
 * defaults.  dense != 0 sizes for dsa_indexer_topk, 0 for dosa_indexer_topk.
 * Returns 0 for invalid arguments. */
size_t dosa_workspace_size(int32_t batch, const int32_t* q_lens, const int32_t* kv_lens,
                           int32_t H, int32_t d, int32_t topk, int32_t q_dtype, int32_t k_dtype,
                           int32_t paged, int32_t dense, const dosa_config* cfg);

/* DoSA path: certificate-pruned exact Top-K.  stats: DEVICE pointer or NULL. */
int dosa_indexer_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                      const void* k, int32_t k_dtype, const float* k_scale,
                      const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
                      const int32_t* page_table, int32_t page_size, int32_t max_pages,
                      int32_t H, int32_t d, int32_t topk,
                      int32_t* out_idx, float* out_score,
                      void* workspace, size_t workspace_bytes,
                      const dosa_config* cfg, dosa_stats* stats, void* stream);

/* Dense path: every visible key scored with all heads, streaming exact Top-K.
 * Of cfg (NULL = defaults) it uses buffer_cap, key_splits and DOSA_SORTED. */
int dsa_indexer_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                     const void* k, int32_t k_dtype, const float* k_scale,
                     const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
                     const int32_t* page_table, int32_t page_size, int32_t max_pages,
                     int32_t H, int32_t d, int32_t topk,
                     int32_t* out_idx, float* out_score,
                     void* workspace, size_t workspace_bytes,
                     const dosa_config* cfg, dosa_stats* stats, void* stream);

/* dosa_indexer_topk without a workspace argument, for callers that cannot
 * allocate device memory (serving loops or harnesses that forbid allocation):
 * the call allocates nothing and runs in a scratch array the library holds
 * in device memory, DOSA_NOALLOC_SCRATCH_BYTES per GPU, reserved when the
 * library's code is loaded on that GPU and kept until the process ends.  The
 * GPU is the device current on the calling thread (the one `stream` belongs
 * to).  A call whose workspace would exceed the scratch size
 * (dosa_workspace_size with dense = 0) returns DOSA_ERR_UNSUPPORTED and
 * enqueues nothing.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on the device (concurrent streams, or other threads) race and
 * must be serialised by the caller; consecutive calls on one stream are safe,
 * and no state carries over from one call to the next.  Arguments, results and
 * errors otherwise as dosa_indexer_topk. */
#define DOSA_NOALLOC_SCRATCH_BYTES (128u << 20)
int dosa_indexer_topk_noalloc(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                              const void* k, int32_t k_dtype, const float* k_scale,
                              const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
                              const int32_t* page_table, int32_t page_size, int32_t max_pages,
                              int32_t H, int32_t d, int32_t topk,
                              int32_t* out_idx, float* out_score,
                              const dosa_config* cfg, dosa_stats* stats, void* stream);

/* Per-pass timing (tracing for benchmarks).  Between dosa_profile_begin()
 * and dosa_profile_end(), every kernel the calling thread enqueues through
 * this library is bracketed by two HIP events recorded on the kernel's own
 * stream.  dosa_profile_end() waits for those events, writes up to
 * max_entries per-pass totals to out (HOST array) and returns the number of
 * entries written, or a negative status.  Off by default; profiling creates
 * HIP event objects (no device memory) and reuses them across sessions.
 * Pass names: prep, key_norms, score_seed, select_seed, plan, bound, compact,
 * score_survivor_tiles, score_survivor_lists, score_dense, select_final. */
typedef struct {
  const char* name;   /* static string */
  int32_t launches;
  double total_ms;    /* sum of the launches' event-to-event durations */
} dosa_kernel_time;

int dosa_profile_begin(void);
int dosa_profile_end(dosa_kernel_time* out, int32_t max_entries);

/* Human-readable text for a status code (static storage; for DOSA_ERR_HIP it
 * names the failing HIP call of the most recent error on this thread). */
const char* dosa_status_string(int status);

/* Library version string. */
const char* dosa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DOSA_INDEXER_H_ */

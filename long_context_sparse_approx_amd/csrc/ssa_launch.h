// Kernel argument blocks and launchers of the stratified sparse decode path.
// Internal to the library: the public interface is include/ssa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

// Which bound ends the deterministic stratum at the current radix digit:
// the count (top-k), the mass (top-p), or both while they share the digit.
enum : int32_t { kBoundCount = 1, kBoundMass = 2 };

// Per-unit facts derived from the first-digit histograms before the chunk
// passes:
//   b1       = first digit of the stratum's last key (2048 when the stratum
//              is empty),
//   rem      = rank of that key among the keys with digit b1 (count bound),
//   rem_mass = mass units still needed within digit b1 (mass bound),
//   mode     = kBoundCount | kBoundMass: the bounds still open at digit b1
//              (0: empty stratum),
//   above    = number of tokens whose first digit is above b1,
//   wlb      = a lower bound of the tail normaliser W (0 when unknown).
struct Thresh1 {
  int32_t b1;
  int32_t rem;
  float wlb;
  int32_t mode;
  unsigned long long rem_mass;
  int32_t above;
  int32_t pad;
};
static_assert(sizeof(Thresh1) == 32, "one 32-byte record per unit");

// The indexer splits the units' token ranges, each rounded up to this many
// tokens, evenly over its workgroups.
constexpr int kIndexAlign = 256;

struct IndexArgs {
  const uint16_t* q;          // [B, T, Hq, d] bf16
  const uint16_t* k_cache;    // [num_blocks, Hkv, 16, key_ld] bf16
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* seq_lens;    // [B]
  float* scores;              // row u of stride score_ld
  int64_t score_ld;
  uint32_t* hist1;            // [U, 2048]
  uint32_t* maxkey;           // [U]
  int T, g, NG;               // queries per sequence, queries per group, groups
  int Hq, Hkv, G, d, pair_begin, pair_count;
  int max_blocks, num_blocks, max_seq_len;
  int units;                  // selection units (score rows)
  int workgroups;             // grid size: the units' tokens are split evenly among them
  int key_ld;                 // elements per key row: d (whole keys) or 2 * pair_count
  int key_off;                // first scored element of a row: 2 * pair_begin or 0
  float scale;
};

// Units: selection units u = (b * NG + grp) * Hkv + h (one per sequence,
// query group and kv head); attention units (b * T + t) * Hkv + h (one per
// query position and kv head).
struct SelectArgs {
  const float* scores;        // row u of stride score_ld
  int64_t score_ld;
  const int32_t* seq_lens;
  const int32_t* topk;
  const float* top_p;         // [B] or null (top-k only)
  const int32_t* sample_budget;
  const uint64_t* seed;
  const float* w_in;          // [U] or null
  const int32_t* block_table; // used when emit_rows
  uint32_t* hist1;            // [U, 2048]
  uint32_t* hist2;            // [U, 2048]
  unsigned long long* hist1m; // [U, 2048] first-digit mass units (top-p)
  unsigned long long* hist2m; // [U, 2048] second-digit mass units of the candidates (top-p)
  uint32_t* maxkey;           // [U]
  Thresh1* thresh;            // [U]
  int32_t* cand_idx;          // [U, seg_ld] threshold-digit candidates per chunk
  uint32_t* cand_key;         // [U, seg_ld]
  float* cand_w;              // [U, seg_ld] the candidates' tail weights sexp(s - M)
  int32_t* cand_cnt;          // [U, nchunk]
  int32_t* list_idx;          // [U, seg_ld] per chunk: above-threshold tokens, then
  float* list_w;              //   sampling candidates with their tail weights
  int32_t* list_cnt;          // [U, nchunk, 2] (n_above, n_sampling_candidates)
  double* wpart;              // [U, nchunk]
  int32_t* tiecnt;            // [U, nchunk]
  int32_t* ties_before;       // [U, nchunk]
  void* state;                // [U] UnitState
  int32_t* sel_idx;           // [U, seg_ld]: positions, or cache rows when emit_rows
  float* sel_logw;            // [U, seg_ld]
  int32_t* sel_cnt;           // [U, nchunk, 2]
  float* norm_out;            // [U, 2] or null
  int max_topk;               // topk[b] above it acts as it (INT_MAX: no bound)
  int kmult;                  // the stratum holds kmult * topk tokens (refine mode's list)
  double* w64;                // [U] the tail sum W in float64, or null
  // Early stopping (all null when it is off).  A stratum word is
  // ((~key) << 32) | position: ascending words are the stratum's order.
  float stop_tau;                 // the threshold tau, clamped to 1
  unsigned long long* stop_cut;   // [U] the last word kept (~0: nothing cut)
  int32_t* stop_off;              // [U, nchunk] offset of each chunk's words above the
                                  //   threshold key in stop_words
  int32_t* stop_n;                // [U] words above the threshold key (<= 16384 when cut)
  unsigned long long* stop_words; // [U, 16384] those words, then sorted per 1024-word slice
  uint16_t* stop_pair;            // [U, 16, 16, 1024] words of slice s below word i of slice o
  unsigned long long* stop_rword; // [U, 16384] the stratum's words in its order (ties too)
  float* stop_logit;              // [U, 16384, 16] exact logit of (rank, query row);
                                  //   -inf outside the row's span
  uint32_t* stop_mkey;            // [U, 256, 16] each 64-token block's largest logit per
                                  //   row (order key; 0: none)
  unsigned long long* stop_gain;  // [U, 256, 16] each 64-token block's gain per row, in units
  // What the exact logits read: the unit's query rows (each member's G
  // heads) and its keys, whole or split, through the block table.
  const uint16_t* q;              // [B, T, Hq, d]
  const uint16_t* k_cache;        // whole keys [rows, d], or the scored dims [rows, 2 pc]
  const uint16_t* k_rest;         // split keys: the other dims; else null
  int Hq, G, d, pair_begin, pair_count;
  float scale;
  int T, g, NG;
  int Hkv, max_seq_len, nchunk, max_blocks, num_blocks, emit_rows;
  int64_t seg_ld;             // nchunk * 4096
};

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k_cache;    // whole keys [rows, d], or the scored dims [rows, 2 * pair_count]
  const uint16_t* k_rest;     // split keys: the other dims [rows, d - 2 * pair_count]; else null
  const uint16_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel_idx;     // positions, or cache rows when idx_are_rows
  const float* sel_logw;
  const int32_t* sel_cnt;
  float* part;                // [B*T*Hq, nsplit * nsub, d + 2]: acc[d], m, l
  void* out;                  // [B, T, Hq, d]
  int T, g, NG;
  int mpw, mblocks;           // members per attention wave (16 / G), waves per group
  int B, Hq, Hkv, G, d, max_blocks, num_blocks, max_seq_len, nchunk, nsplit, out_dtype;
  int nsub;                   // waves per split, each taking an equal share of every chunk's
                              //   items; partial states per query row: nsplit * nsub
  int idx_are_rows;
  int pair_begin, pair_count; // the scored dims, for split keys
  int64_t seg_ld;
  float scale;
  // Selection taken by the attention waves (no early stop, no refine): the
  // selection stage's per-chunk lists and unit states replace
  // sel_idx / sel_logw / sel_cnt, and the sample kernel is not run.
  int fused_select;
  const int32_t* list_idx;    // as in SelectArgs
  const float* list_w;
  const int32_t* list_cnt;
  const int32_t* cand_idx;
  const uint32_t* cand_key;
  const float* cand_w;
  const int32_t* cand_cnt;
  const int32_t* tiecnt;
  const int32_t* ties_before;
  const void* state;          // [U] UnitState
  const uint64_t* seed;
  float* sel_scratch;         // [U, seg_ld]: a sampled position's logit bias, for chunks
                              //   whose lists exceed what the waves hold in registers
};

// Refine mode of query groups: every member re-ranks the group's candidate
// list (the group selection's deterministic entries) by its own score.
// Member units are v = (b * T + t) * Hkv + h.
struct RefineArgs {
  const float* scores;        // the group's proxy scores, row u of stride score_ld
  int64_t score_ld;
  const int32_t* gsel_idx;    // [U, seg_ld] the group selection (positions)
  const int32_t* gsel_cnt;    // [U, nchunk, 2]
  const void* gstate;         // [U] UnitState of the group selection
  const double* gw64;         // [U] the group's tail sum (its span minus C), float64
  const int32_t* seq_lens;
  const int32_t* topk;
  const int32_t* sample_budget;
  const uint64_t* seed;
  const float* w_in;          // [Um] replaces each member's normaliser, or null
  const uint16_t* q;          // [B, T, Hq, d]
  const uint16_t* k_cache;    // the scored dims of row r at k_cache + r * key_ld + key_off
  const int32_t* block_table;
  uint32_t* own_key;          // [Um, seg_ld] member's order key of each group entry
  float* cand_pw;             // [U, seg_ld] proxy weight sexp(s - M) of each group candidate
  void* mstate;               // [Um] MemberState
  int32_t* msel_idx;          // [Um, seg_ld] member selections (positions)
  float* msel_logw;           // [Um, seg_ld]
  int32_t* msel_cnt;          // [Um, nchunk, 2]
  float* norm_out;            // [Um, 2] (M, W_t) or null
  int T, g, NG, Hq, Hkv, G, d, pair_begin, pair_count;
  int max_seq_len, nchunk, max_blocks, num_blocks, max_topk;
  int key_ld, key_off;
  int64_t seg_ld;
  float own_scale;            // fl32(fl32(scale) / G)
};

// Appending new tokens' keys and values to the cache (whole or split keys).
struct AppendArgs {
  const uint16_t* k_new;      // [B, T, Hkv, d]
  const uint16_t* v_new;      // [B, T, Hkv, d]
  const int32_t* block_table; // [B, max_blocks]
  const int32_t* seq_lens;    // [B], lengths including the new tokens
  uint16_t* k_cache;          // whole keys, or the scored dims when k_rest is set
  uint16_t* k_rest;           // the other dims, or null
  uint16_t* v_cache;
  int B, T, Hkv, d, pair_begin, pair_count, max_blocks, num_blocks, max_seq_len;
};

int indexer_resident_workgroups(int pair_count);  // 0 if unknown
// Clears the histograms and maxima; the mass histograms only when non-null.
hipError_t launch_init(uint32_t* hist1, uint32_t* hist2, uint32_t* maxkey,
                       unsigned long long* hist1m, unsigned long long* hist2m, int units,
                       hipStream_t stream);
hipError_t launch_indexer(const IndexArgs& a, int units, hipStream_t stream);
hipError_t launch_score_hist(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_mass(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_threshold(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_filter(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_resolve(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_stop(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_sample(const SelectArgs& a, int units, hipStream_t stream);
hipError_t launch_attend(const AttendArgs& a, hipStream_t stream);
// The attention stage taking the sample stage's decisions itself (fused_select).
hipError_t launch_attend_select(const AttendArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_refine(const RefineArgs& a, int group_units, int member_units,
                         hipStream_t stream);
hipError_t launch_merge(const AttendArgs& a, hipStream_t stream);
hipError_t launch_debug_philox(uint64_t seed, int b, int h, int grp, int j0, int n,
                               uint32_t* words, hipStream_t stream);
hipError_t launch_debug_sexp(const float* x, float* y, int n, hipStream_t stream);
hipError_t launch_debug_tail_exp(const float* x, float* y, int n, hipStream_t stream);

}  // namespace ssa

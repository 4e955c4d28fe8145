// Host side of the C ABI declared in include/ssa.h: argument validation,
// workspace carving and the launch sequence of each entry point.  No
// allocation, no synchronisation, no global mutable state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "ssa.h"
#include "ssa_launch.h"

namespace {

struct UnitStateBytes {
  uint32_t words[8];  // layout of ssa::UnitState (32 bytes)
};

constexpr size_t kAlign = 256;
constexpr int kBins = 2048;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool params_ok(const ssa_params* p) {
  if (!p) return false;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1) return false;
  if (p->num_q_heads % p->num_kv_heads != 0) return false;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > 16) return false;
  if (p->head_dim != 64 && p->head_dim != 128) return false;
  if (p->block_size != SSA_BLOCK_TOKENS) return false;
  if (p->max_blocks_per_seq < 1 || p->num_blocks < 1) return false;
  if (p->max_seq_len < 1 || p->max_seq_len > SSA_MAX_SEQ_LEN) return false;
  if ((int64_t)p->max_seq_len > (int64_t)p->max_blocks_per_seq * SSA_BLOCK_TOKENS) return false;
  // cache rows are addressed with 32-bit row numbers
  if ((int64_t)p->num_blocks * p->num_kv_heads * SSA_BLOCK_TOKENS >= ((int64_t)1 << 31)) return false;
  const int pc = p->pair_count;
  if (pc != 4 && pc != 8 && pc != 16 && pc != 32 && pc != 64) return false;
  if (p->pair_begin < 0 || p->pair_begin % 4 != 0) return false;
  if (p->pair_begin + pc > p->head_dim / 2) return false;
  if (p->num_splits < 0) return false;
  if (p->out_dtype != SSA_F32 && p->out_dtype != SSA_BF16) return false;
  if (!(p->softmax_scale >= 0.0f) || !std::isfinite(p->softmax_scale)) return false;
  if (p->num_queries < 1 || p->num_queries > 256 || p->query_group < 1) return false;
  if (p->key_layout != SSA_KEYS_WHOLE && p->key_layout != SSA_KEYS_SPLIT) return false;
  if (p->max_topk < 0 || p->refine < 0) return false;
  if (p->refine > 0) {
    if (p->early_stop > 0.0f) return false;  // not combined with early stopping
    // the refine kernels stage the group's scored query slices in LDS
    const int g = p->query_group < p->num_queries ? p->query_group : p->num_queries;
    if ((int64_t)g * G * 2 * p->pair_count > 8192) return false;
  }
  if (p->early_stop > 0.0f) {  // NaN compares false: off
    // the stratum must fit the early-stopping kernels, and so must the rows
    const int bound = p->max_topk > 0 ? p->max_topk : p->max_seq_len;
    if (bound > SSA_STOP_MAX_STRATUM) return false;
    const int g = p->query_group < p->num_queries ? p->query_group : p->num_queries;
    if ((int64_t)g * G > SSA_STOP_MAX_ROWS) return false;
  }
  const int64_t ng = (p->num_queries + p->query_group - 1) / p->query_group;
  // grid.y of the per-unit and per-(query position, kv head) launches
  if ((int64_t)p->batch * ng * p->num_kv_heads > 65535) return false;
  // attention: one wave per (selection unit, block of 16 / G members)
  {
    const int G = p->num_q_heads / p->num_kv_heads;
    const int g = p->query_group < p->num_queries ? p->query_group : p->num_queries;
    const int64_t mblocks = (g + 16 / G - 1) / (16 / G);
    if ((int64_t)p->batch * ng * p->num_kv_heads * mblocks > 65535) return false;
  }
  return true;
}

struct Dims {
  int B, Hq, Hkv, G, d, T, g, NG, U, NC, NS;
  int refine;  // candidate list factor r of the refine mode (0: reuse)
  int Um;      // member units B * T * Hkv (refine mode)
  int NSUB;  // attention waves per split (NS * NSUB <= the merge's 4096 states)
  int64_t SEG;
  float scale;
  bool stop;  // early stopping on (its buffers are part of the workspace)
};

// Attention waves per split: each takes an equal share of every chunk's
// selected items (a chunk holds about 82 of them at 50x sparsity, 3 tiles of
// 32), which shortens each wave's chain of dependent loads, and the merge
// reads that many more partial states.  Measured: more waves help while the
// launch has fewer than about 2048 (128K x 4: 1024 waves -> 2 per split, the
// attention 18.7 -> 15.6 us) and cost beyond (1M: 2048 waves; 2 per split
// 23.7 -> 26.4 us).
constexpr int kAttendWaves = 2048;
constexpr int kAttendMaxSub = 4;

Dims dims_of(const ssa_params* p) {
  Dims d;
  d.B = p->batch;
  d.Hq = p->num_q_heads;
  d.Hkv = p->num_kv_heads;
  d.G = d.Hq / d.Hkv;
  d.d = p->head_dim;
  d.T = p->num_queries;
  d.g = p->query_group < p->num_queries ? p->query_group : p->num_queries;
  d.NG = (d.T + d.g - 1) / d.g;
  d.U = d.B * d.NG * d.Hkv;  // selection units
  d.NC = (p->max_seq_len + SSA_CHUNK_TOKENS - 1) / SSA_CHUNK_TOKENS;
  d.SEG = (int64_t)d.NC * SSA_CHUNK_TOKENS;
  d.NS = p->num_splits == 0 ? d.NC : (p->num_splits < d.NC ? p->num_splits : d.NC);
  d.refine = p->refine;
  d.Um = d.B * d.T * d.Hkv;
  {
    // Attention runs over the selection units, or with refine over the
    // member units (one member each).
    const int ag = d.refine > 0 ? 1 : d.g;
    const int64_t au = d.refine > 0 ? d.Um : d.U;
    const int mpw = 16 / d.G;  // query columns per attention wave: members x heads
    const int64_t waves = (int64_t)d.NS * au * ((ag + mpw - 1) / mpw);
    d.NSUB = 1;
    while (d.NSUB < kAttendMaxSub && waves * d.NSUB * 2 <= kAttendWaves &&
           (int64_t)d.NS * d.NSUB * 2 <= SSA_MAX_SEQ_LEN / SSA_CHUNK_TOKENS)
      d.NSUB *= 2;
  }
  d.scale = p->softmax_scale > 0.0f ? p->softmax_scale
                                     : (float)(1.0 / std::sqrt((double)p->head_dim));
  d.stop = p->early_stop > 0.0f;  // NaN compares false
  return d;
}

struct Layout {
  size_t scores, hist1, hist2, hist1m, hist2m, maxkey, thresh, cand_idx, cand_key, cand_w, cand_cnt,
      list_idx, list_w,
      list_cnt, wpart, tiecnt,
      ties_before, state, sel_idx, sel_logw, sel_cnt, part, stop_cut, stop_off, stop_n,
      stop_words, stop_pair, stop_rword, stop_logit, stop_mkey, stop_gain, w64, own_key, cand_pw, mstate, msel_idx, msel_logw,
      msel_cnt, total;
};

Layout layout_of(const Dims& d) {
  Layout l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t U = (size_t)d.U, SEG = (size_t)d.SEG, NC = (size_t)d.NC;
  l.scores = take(U * SEG * 4);
  l.hist1 = take(U * kBins * 4);
  l.hist2 = take(U * kBins * 4);
  l.hist1m = take(U * kBins * 8);
  l.hist2m = take(U * kBins * 8);
  l.maxkey = take(U * 4);
  l.thresh = take(U * sizeof(ssa::Thresh1));
  l.cand_idx = take(U * SEG * 4);
  l.cand_key = take(U * SEG * 4);
  l.cand_w = take(U * SEG * 4);
  l.cand_cnt = take(U * NC * 4);
  l.list_idx = take(U * SEG * 4);
  l.list_w = take(U * SEG * 4);
  l.list_cnt = take(U * NC * 2 * 4);
  l.wpart = take(U * NC * 8);
  l.tiecnt = take(U * NC * 4);
  l.ties_before = take(U * NC * 4);
  l.state = take(U * sizeof(UnitStateBytes));
  l.sel_idx = take(U * SEG * 4);
  l.sel_logw = take(U * SEG * 4);
  l.sel_cnt = take(U * NC * 2 * 4);
  l.part = take((size_t)d.B * d.T * d.Hq * d.NS * d.NSUB * (d.d + 2) * 4);
  const size_t SU = d.stop ? U : 0;  // early stopping's buffers only when it is on
  const size_t KS = SSA_STOP_MAX_STRATUM;
  l.stop_cut = take(SU * 8);
  l.stop_off = take(SU * NC * 4);
  l.stop_n = take(SU * 4);
  l.stop_words = take(SU * KS * 8);
  l.stop_pair = take(SU * (KS / 1024) * (KS / 1024) * 1024 * 2);
  l.stop_rword = take(SU * KS * 8);
  l.stop_logit = take(SU * KS * SSA_STOP_MAX_ROWS * 4);
  l.stop_mkey = take(SU * (KS / 64) * SSA_STOP_MAX_ROWS * 4);
  l.stop_gain = take(SU * (KS / 64) * SSA_STOP_MAX_ROWS * 8);
  // refine mode's member selections (only when it is on)
  const size_t RU = d.refine > 0 ? (size_t)d.U : 0;
  const size_t RM = d.refine > 0 ? (size_t)d.Um : 0;
  l.w64 = take(RU * 8);
  l.own_key = take(RM * SEG * 4);
  l.cand_pw = take(RU * SEG * 4);
  l.mstate = take(RM * 32);
  l.msel_idx = take(RM * SEG * 4);
  l.msel_logw = take(RM * SEG * 4);
  l.msel_cnt = take(RM * NC * 2 * 4);
  l.total = off;
  return l;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

struct Recorder {
  void* const* ev;
  hipStream_t s;
  void begin(int stage) const {
    if (ev && ev[2 * stage]) (void)hipEventRecord((hipEvent_t)ev[2 * stage], s);
  }
  void end(int stage) const {
    if (ev && ev[2 * stage + 1]) (void)hipEventRecord((hipEvent_t)ev[2 * stage + 1], s);
  }
};

// The indexer's grid: as many workgroups as the device holds at once, so the
// layer's tokens (split evenly among them) stream in a single round; never
// more than the units' longest possible token ranges have aligned blocks.
int indexer_workgroups(const ssa_params* p, const Dims& d) {
  const int resident = ssa::indexer_resident_workgroups(p->pair_count);
  const int64_t blocks =
      (int64_t)d.U * ((p->max_seq_len + ssa::kIndexAlign - 1) / ssa::kIndexAlign);
  const int64_t g = resident > 0 ? resident : 1024;
  return (int)(blocks < 1 ? 1 : (blocks < g ? blocks : g));
}

ssa::IndexArgs index_args(const ssa_params* p, const Dims& d, const void* q, const void* k_cache,
                          const int32_t* block_table, const int32_t* seq_lens, float* scores,
                          int64_t score_ld, void* ws, const Layout& l) {
  ssa::IndexArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.scores = scores;
  a.score_ld = score_ld;
  a.hist1 = at<uint32_t>(ws, l.hist1);
  a.maxkey = at<uint32_t>(ws, l.maxkey);
  a.T = d.T;
  a.g = d.g;
  a.NG = d.NG;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.d = d.d;
  a.pair_begin = p->pair_begin;
  a.pair_count = p->pair_count;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.max_seq_len = p->max_seq_len;
  a.units = d.U;
  a.workgroups = indexer_workgroups(p, d);
  const bool split = p->key_layout == SSA_KEYS_SPLIT;
  a.key_ld = split ? 2 * p->pair_count : d.d;
  a.key_off = split ? 0 : 2 * p->pair_begin;
  a.scale = d.scale;
  return a;
}

// Keys as the kernels take them: whole rows (rest null), or the scored dims
// and the others.
struct Keys {
  const void* main;
  const void* rest;
};

ssa::SelectArgs select_args(const ssa_params* p, const Dims& d, const float* scores,
                            int64_t score_ld, const int32_t* seq_lens, const int32_t* topk,
                            const float* top_p, const int32_t* sample_budget,
                            const uint64_t* seed, const float* w_in, const void* q, Keys keys,
                            const int32_t* block_table, int emit_rows, int32_t* sel_idx,
                            float* sel_logw, int32_t* sel_cnt, float* norm_out, void* ws,
                            const Layout& l) {
  ssa::SelectArgs a;
  a.scores = scores;
  a.score_ld = score_ld;
  a.seq_lens = seq_lens;
  a.topk = topk;
  a.top_p = top_p;
  a.sample_budget = sample_budget;
  a.seed = seed;
  a.w_in = w_in;
  a.block_table = block_table;
  a.hist1 = at<uint32_t>(ws, l.hist1);
  a.hist2 = at<uint32_t>(ws, l.hist2);
  a.hist1m = at<unsigned long long>(ws, l.hist1m);
  a.hist2m = at<unsigned long long>(ws, l.hist2m);
  a.maxkey = at<uint32_t>(ws, l.maxkey);
  a.thresh = at<ssa::Thresh1>(ws, l.thresh);
  a.cand_idx = at<int32_t>(ws, l.cand_idx);
  a.cand_key = at<uint32_t>(ws, l.cand_key);
  a.cand_w = at<float>(ws, l.cand_w);
  a.cand_cnt = at<int32_t>(ws, l.cand_cnt);
  a.list_idx = at<int32_t>(ws, l.list_idx);
  a.list_w = at<float>(ws, l.list_w);
  a.list_cnt = at<int32_t>(ws, l.list_cnt);
  a.wpart = at<double>(ws, l.wpart);
  a.tiecnt = at<int32_t>(ws, l.tiecnt);
  a.ties_before = at<int32_t>(ws, l.ties_before);
  a.state = at<void>(ws, l.state);
  a.sel_idx = sel_idx;
  a.sel_logw = sel_logw;
  a.sel_cnt = sel_cnt;
  a.norm_out = norm_out;
  // early stopping is on for tau > 0 (NaN compares false)
  a.stop_tau = p->early_stop > 1.0f ? 1.0f : p->early_stop;
  a.stop_cut = d.stop ? at<unsigned long long>(ws, l.stop_cut) : nullptr;
  a.stop_off = d.stop ? at<int32_t>(ws, l.stop_off) : nullptr;
  a.stop_n = d.stop ? at<int32_t>(ws, l.stop_n) : nullptr;
  a.stop_words = d.stop ? at<unsigned long long>(ws, l.stop_words) : nullptr;
  a.stop_pair = d.stop ? at<uint16_t>(ws, l.stop_pair) : nullptr;
  a.stop_rword = d.stop ? at<unsigned long long>(ws, l.stop_rword) : nullptr;
  a.stop_logit = d.stop ? at<float>(ws, l.stop_logit) : nullptr;
  a.stop_mkey = d.stop ? at<uint32_t>(ws, l.stop_mkey) : nullptr;
  a.stop_gain = d.stop ? at<unsigned long long>(ws, l.stop_gain) : nullptr;
  a.max_topk = p->max_topk > 0 ? p->max_topk : INT32_MAX;
  a.kmult = d.refine > 0 ? d.refine : 1;
  a.w64 = d.refine > 0 ? at<double>(ws, l.w64) : nullptr;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(keys.main);
  a.k_rest = static_cast<const uint16_t*>(keys.rest);
  a.Hq = d.Hq;
  a.G = d.G;
  a.d = d.d;
  a.pair_begin = p->pair_begin;
  a.pair_count = p->pair_count;
  a.scale = d.scale;
  a.T = d.T;
  a.g = d.g;
  a.NG = d.NG;
  a.Hkv = d.Hkv;
  a.max_seq_len = p->max_seq_len;
  a.nchunk = d.NC;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.emit_rows = emit_rows;
  a.seg_ld = d.SEG;
  return a;
}

// The refine stage: the group selection (sel_*) is refined into member
// selections (msel_*); norm_out and w_in are per member unit.
ssa::RefineArgs refine_args(const ssa_params* p, const Dims& d, const ssa::SelectArgs& sa,
                            const void* q, const void* k_main, const int32_t* block_table,
                            const float* w_in, int32_t* msel_idx, float* msel_logw,
                            int32_t* msel_cnt, float* norm_out, void* ws, const Layout& l) {
  ssa::RefineArgs r;
  r.scores = sa.scores;
  r.score_ld = sa.score_ld;
  r.gsel_idx = sa.sel_idx;
  r.gsel_cnt = sa.sel_cnt;
  r.gstate = sa.state;
  r.gw64 = at<double>(ws, l.w64);
  r.seq_lens = sa.seq_lens;
  r.topk = sa.topk;
  r.sample_budget = sa.sample_budget;
  r.seed = sa.seed;
  r.w_in = w_in;
  r.q = static_cast<const uint16_t*>(q);
  r.k_cache = static_cast<const uint16_t*>(k_main);
  r.block_table = block_table;
  r.own_key = at<uint32_t>(ws, l.own_key);
  r.cand_pw = at<float>(ws, l.cand_pw);
  r.mstate = at<void>(ws, l.mstate);
  r.msel_idx = msel_idx;
  r.msel_logw = msel_logw;
  r.msel_cnt = msel_cnt;
  r.norm_out = norm_out;
  r.T = d.T;
  r.g = d.g;
  r.NG = d.NG;
  r.Hq = d.Hq;
  r.Hkv = d.Hkv;
  r.G = d.G;
  r.d = d.d;
  r.pair_begin = p->pair_begin;
  r.pair_count = p->pair_count;
  r.max_seq_len = p->max_seq_len;
  r.nchunk = d.NC;
  r.max_blocks = p->max_blocks_per_seq;
  r.num_blocks = p->num_blocks;
  r.max_topk = p->max_topk > 0 ? p->max_topk : INT32_MAX;
  const bool split = p->key_layout == SSA_KEYS_SPLIT;
  r.key_ld = split ? 2 * p->pair_count : d.d;
  r.key_off = split ? 0 : 2 * p->pair_begin;
  r.seg_ld = d.SEG;
  r.own_scale = d.scale / (float)d.G;  // one float32 division
  return r;
}

ssa::AttendArgs attend_args(const ssa_params* p, const Dims& d, const void* q, Keys keys,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* sel_idx, const float* sel_logw,
                            const int32_t* sel_cnt, int idx_are_rows, void* out, void* ws,
                            const Layout& l) {
  ssa::AttendArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(keys.main);
  a.k_rest = static_cast<const uint16_t*>(keys.rest);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.sel_idx = sel_idx;
  a.sel_logw = sel_logw;
  a.sel_cnt = sel_cnt;
  a.part = at<float>(ws, l.part);
  a.out = out;
  a.T = d.T;
  // With refine every member has its own selection: one member per unit.
  a.g = d.refine > 0 ? 1 : d.g;
  a.NG = d.refine > 0 ? d.T : d.NG;
  a.mpw = 16 / d.G;  // G <= 16
  a.mblocks = (a.g + a.mpw - 1) / a.mpw;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.d = d.d;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.max_seq_len = p->max_seq_len;
  a.nchunk = d.NC;
  a.nsplit = d.NS;
  a.nsub = d.NSUB;
  a.out_dtype = p->out_dtype;
  a.idx_are_rows = idx_are_rows;
  a.pair_begin = p->pair_begin;
  a.pair_count = p->pair_count;
  a.seg_ld = d.SEG;
  a.scale = d.scale;
  a.fused_select = 0;
  a.list_idx = nullptr;
  a.list_w = nullptr;
  a.list_cnt = nullptr;
  a.cand_idx = nullptr;
  a.cand_key = nullptr;
  a.cand_w = nullptr;
  a.cand_cnt = nullptr;
  a.tiecnt = nullptr;
  a.ties_before = nullptr;
  a.state = nullptr;
  a.seed = nullptr;
  a.sel_scratch = nullptr;
  return a;
}

// The attention stage takes the sample stage's decisions from the selection
// stage's lists (no early stop, no refine); the position-indexed
// scratch row is the selection's bias array, which nothing else reads then.
void fuse_select(ssa::AttendArgs* a, const ssa::SelectArgs& s) {
  a->fused_select = 1;
  a->list_idx = s.list_idx;
  a->list_w = s.list_w;
  a->list_cnt = s.list_cnt;
  a->cand_idx = s.cand_idx;
  a->cand_key = s.cand_key;
  a->cand_w = s.cand_w;
  a->cand_cnt = s.cand_cnt;
  a->tiecnt = s.tiecnt;
  a->ties_before = s.ties_before;
  a->state = s.state;
  a->seed = s.seed;
  a->sel_scratch = s.sel_logw;
}

#define SSA_TRY(expr)                        \
  do {                                       \
    if ((expr) != hipSuccess) return SSA_ERR_HIP; \
  } while (0)

// The selection stages of both entry points: clear, first-digit histogram
// (fused into the indexer in ssa_decode), top-p mass histogram when asked
// for, threshold, filter.
hipError_t launch_init_for(const ssa::SelectArgs& a, int units, hipStream_t s) {
  const bool topp = a.top_p != nullptr;
  return ssa::launch_init(a.hist1, a.hist2, a.maxkey, topp ? a.hist1m : nullptr,
                          topp ? a.hist2m : nullptr, units, s);
}

// The resolve stage, then the early-stopping cut when it is on.
hipError_t launch_resolve_for(const ssa::SelectArgs& a, int units, hipStream_t s) {
  const hipError_t e = ssa::launch_resolve(a, units, s);
  if (e != hipSuccess || !a.stop_cut) return e;
  return ssa::launch_stop(a, units, s);
}

hipError_t launch_first_digit(const ssa::SelectArgs& a, int units, hipStream_t s) {
  if (a.top_p) {
    const hipError_t e = ssa::launch_mass(a, units, s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = ssa::launch_threshold(a, units, s);
  if (e != hipSuccess) return e;
  return ssa::launch_filter(a, units, s);
}

int check_ws(const ssa_params* p, void* ws, size_t ws_bytes, Layout* l) {
  if (!params_ok(p)) return SSA_ERR_INVALID;
  *l = layout_of(dims_of(p));
  if (!ws || !aligned16(ws)) return SSA_ERR_INVALID;
  if (ws_bytes < l->total) return SSA_ERR_WORKSPACE;
  return SSA_OK;
}

// Split keys need the rest array unless the scored dims are the whole head.
bool split_keys_ok(const ssa_params* p, const void* k_dom, const void* k_rest) {
  if (p->key_layout != SSA_KEYS_SPLIT || !k_dom || !aligned16(k_dom)) return false;
  if (2 * p->pair_count == p->head_dim) return true;
  return k_rest && aligned16(k_rest);
}

// Rest array as the kernels take it: null when there are no rest dims.
const void* rest_of(const ssa_params* p, const void* k_rest) {
  return 2 * p->pair_count == p->head_dim ? nullptr : k_rest;
}

int decode_impl(const ssa_params* p, const void* q, Keys keys, const void* v_cache,
                const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk,
                const float* top_p, const int32_t* sample_budget, const uint64_t* seed, void* out,
                void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  Layout l;
  const int rc = check_ws(p, workspace, workspace_bytes, &l);
  if (rc != SSA_OK) return rc;
  if (!q || !keys.main || !v_cache || !block_table || !seq_lens || !topk || !sample_budget ||
      !seed || !out)
    return SSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(keys.main) || !aligned16(v_cache)) return SSA_ERR_INVALID;
  const Dims d = dims_of(p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Recorder rec{events, s};
  float* scores = at<float>(workspace, l.scores);
  int32_t* sel_idx = at<int32_t>(workspace, l.sel_idx);
  float* sel_logw = at<float>(workspace, l.sel_logw);
  int32_t* sel_cnt = at<int32_t>(workspace, l.sel_cnt);

  const ssa::IndexArgs ia =
      index_args(p, d, q, keys.main, block_table, seq_lens, scores, d.SEG, workspace, l);
  // One query per sequence: the selection can hold cache rows (one dependent
  // load less in the gather).  Several: positions, so that every member
  // applies its own causal span.
  if (d.refine > 0 && top_p) return SSA_ERR_INVALID;  // refine ranks by count only
  const int rows = d.T == 1 && d.refine == 0 ? 1 : 0;
  const ssa::SelectArgs sa =
      select_args(p, d, scores, d.SEG, seq_lens, topk, top_p, sample_budget, seed, nullptr, q,
                  keys, block_table, rows, sel_idx, sel_logw, sel_cnt, nullptr, workspace, l);
  // With refine, attention reads the member selections.
  int32_t* a_idx = sel_idx;
  float* a_logw = sel_logw;
  int32_t* a_cnt = sel_cnt;
  ssa::RefineArgs ra{};
  if (d.refine > 0) {
    a_idx = at<int32_t>(workspace, l.msel_idx);
    a_logw = at<float>(workspace, l.msel_logw);
    a_cnt = at<int32_t>(workspace, l.msel_cnt);
    ra = refine_args(p, d, sa, q, keys.main, block_table, nullptr, a_idx, a_logw, a_cnt, nullptr,
                     workspace, l);
  }
  ssa::AttendArgs aa = attend_args(p, d, q, keys, v_cache, block_table, seq_lens, a_idx, a_logw,
                                   a_cnt, rows, out, workspace, l);
  const bool fused = d.refine == 0 && !sa.stop_cut;
  if (fused) fuse_select(&aa, sa);
  rec.begin(SSA_STAGE_INIT);
  SSA_TRY(launch_init_for(sa, d.U, s));
  rec.end(SSA_STAGE_INIT);
  rec.begin(SSA_STAGE_INDEX);
  SSA_TRY(ssa::launch_indexer(ia, d.U, s));
  rec.end(SSA_STAGE_INDEX);
  rec.begin(SSA_STAGE_FILTER);
  SSA_TRY(launch_first_digit(sa, d.U, s));
  rec.end(SSA_STAGE_FILTER);
  rec.begin(SSA_STAGE_RESOLVE);
  SSA_TRY(launch_resolve_for(sa, d.U, s));
  rec.end(SSA_STAGE_RESOLVE);
  rec.begin(SSA_STAGE_SAMPLE);
  if (!fused) SSA_TRY(ssa::launch_sample(sa, d.U, s));
  if (d.refine > 0) SSA_TRY(ssa::launch_refine(ra, d.U, d.Um, s));
  rec.end(SSA_STAGE_SAMPLE);
  rec.begin(SSA_STAGE_ATTEND);
  SSA_TRY(fused ? ssa::launch_attend_select(aa, s) : ssa::launch_attend(aa, s));
  rec.end(SSA_STAGE_ATTEND);
  rec.begin(SSA_STAGE_MERGE);
  SSA_TRY(ssa::launch_merge(aa, s));
  rec.end(SSA_STAGE_MERGE);
  return SSA_OK;
}

int attend_impl(const ssa_params* p, const void* q, Keys keys, const void* v_cache,
                const int32_t* block_table, const int32_t* seq_lens, const int32_t* sel_idx,
                const float* sel_logw, const int32_t* sel_count, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  Layout l;
  const int rc = check_ws(p, workspace, workspace_bytes, &l);
  if (rc != SSA_OK) return rc;
  if (!q || !keys.main || !v_cache || !block_table || !seq_lens || !sel_idx || !sel_logw ||
      !sel_count || !out)
    return SSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(keys.main) || !aligned16(v_cache)) return SSA_ERR_INVALID;
  const Dims d = dims_of(p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ssa::AttendArgs aa = attend_args(p, d, q, keys, v_cache, block_table, seq_lens, sel_idx,
                                         sel_logw, sel_count, /*idx_are_rows=*/0, out, workspace,
                                         l);
  SSA_TRY(ssa::launch_attend(aa, s));
  SSA_TRY(ssa::launch_merge(aa, s));
  return SSA_OK;
}

}  // namespace

extern "C" {

size_t ssa_workspace_bytes(const ssa_params* p) {
  if (!params_ok(p)) return 0;
  return layout_of(dims_of(p)).total;
}

int32_t ssa_num_chunks(const ssa_params* p) {
  if (!params_ok(p)) return 0;
  return dims_of(p).NC;
}

int ssa_decode_timed(const ssa_params* p, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk,
                     const float* top_p, const int32_t* sample_budget, const uint64_t* seed,
                     void* out, void* workspace, size_t workspace_bytes, void* stream,
                     void* const* events) {
  if (!p || p->key_layout != SSA_KEYS_WHOLE) return SSA_ERR_INVALID;
  return decode_impl(p, q, Keys{k_cache, nullptr}, v_cache, block_table, seq_lens, topk, top_p,
                     sample_budget, seed, out, workspace, workspace_bytes, stream, events);
}

int ssa_decode_split(const ssa_params* p, const void* q, const void* k_dom, const void* k_rest,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* topk, const float* top_p, const int32_t* sample_budget,
                     const uint64_t* seed, void* out, void* workspace, size_t workspace_bytes,
                     void* stream, void* const* events) {
  if (!params_ok(p) || !split_keys_ok(p, k_dom, k_rest)) return SSA_ERR_INVALID;
  return decode_impl(p, q, Keys{k_dom, rest_of(p, k_rest)}, v_cache, block_table, seq_lens, topk,
                     top_p, sample_budget, seed, out, workspace, workspace_bytes, stream, events);
}

int ssa_decode(const ssa_params* p, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk,
               const float* top_p, const int32_t* sample_budget, const uint64_t* seed, void* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  return ssa_decode_timed(p, q, k_cache, v_cache, block_table, seq_lens, topk, top_p,
                          sample_budget, seed, out, workspace, workspace_bytes, stream, nullptr);
}

int ssa_score(const ssa_params* p, const void* q, const void* k_cache, const int32_t* block_table,
              const int32_t* seq_lens, float* scores, void* workspace, size_t workspace_bytes,
              void* stream) {
  Layout l;
  const int rc = check_ws(p, workspace, workspace_bytes, &l);
  if (rc != SSA_OK) return rc;
  if (!q || !k_cache || !block_table || !seq_lens || !scores) return SSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_cache)) return SSA_ERR_INVALID;
  const Dims d = dims_of(p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ssa::IndexArgs ia = index_args(p, d, q, k_cache, block_table, seq_lens, scores,
                                       p->max_seq_len, workspace, l);
  SSA_TRY(ssa::launch_init(ia.hist1, at<uint32_t>(workspace, l.hist2), ia.maxkey, nullptr,
                           nullptr, d.U, s));
  SSA_TRY(ssa::launch_indexer(ia, d.U, s));
  return SSA_OK;
}

int ssa_select(const ssa_params* p, const float* scores, const int32_t* seq_lens,
               const int32_t* topk, const float* top_p, const int32_t* sample_budget,
               const uint64_t* seed, const float* w_in, const void* q, const void* k_cache,
               const void* k_rest, const int32_t* block_table, int32_t* sel_idx, float* sel_logw,
               int32_t* sel_count, float* norm_out, void* workspace, size_t workspace_bytes,
               void* stream) {
  Layout l;
  const int rc = check_ws(p, workspace, workspace_bytes, &l);
  if (rc != SSA_OK) return rc;
  if (!scores || !seq_lens || !topk || !sample_budget || !seed || !sel_idx || !sel_logw ||
      !sel_count || !norm_out)
    return SSA_ERR_INVALID;
  const Dims d = dims_of(p);
  Keys keys{nullptr, nullptr};
  if (d.refine > 0 && top_p) return SSA_ERR_INVALID;  // refine ranks by count only
  if (d.stop || d.refine > 0) {  // exact gains and own scores read the query and keys
    if (!q || !aligned16(q) || !block_table) return SSA_ERR_INVALID;
    if (p->key_layout == SSA_KEYS_SPLIT) {
      if (!split_keys_ok(p, k_cache, k_rest)) return SSA_ERR_INVALID;
      keys = Keys{k_cache, rest_of(p, k_rest)};
    } else {
      if (!k_cache || !aligned16(k_cache) || k_rest) return SSA_ERR_INVALID;
      keys = Keys{k_cache, nullptr};
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.refine > 0) {
    // The group selection goes to the workspace, the members' to the caller.
    const ssa::SelectArgs sa = select_args(
        p, d, scores, p->max_seq_len, seq_lens, topk, nullptr, sample_budget, seed, nullptr, q,
        keys, block_table, /*emit_rows=*/0, at<int32_t>(workspace, l.sel_idx),
        at<float>(workspace, l.sel_logw), at<int32_t>(workspace, l.sel_cnt), nullptr,
        workspace, l);
    const ssa::RefineArgs ra = refine_args(p, d, sa, q, keys.main, block_table, w_in, sel_idx,
                                           sel_logw, sel_count, norm_out, workspace, l);
    SSA_TRY(launch_init_for(sa, d.U, s));
    SSA_TRY(ssa::launch_score_hist(sa, d.U, s));
    SSA_TRY(launch_first_digit(sa, d.U, s));
    SSA_TRY(launch_resolve_for(sa, d.U, s));
    SSA_TRY(ssa::launch_sample(sa, d.U, s));
    SSA_TRY(ssa::launch_refine(ra, d.U, d.Um, s));
    return SSA_OK;
  }
  const ssa::SelectArgs sa =
      select_args(p, d, scores, p->max_seq_len, seq_lens, topk, top_p, sample_budget, seed, w_in,
                  q, keys, block_table, /*emit_rows=*/0, sel_idx, sel_logw, sel_count, norm_out,
                  workspace, l);
  SSA_TRY(launch_init_for(sa, d.U, s));
  SSA_TRY(ssa::launch_score_hist(sa, d.U, s));
  SSA_TRY(launch_first_digit(sa, d.U, s));
  SSA_TRY(launch_resolve_for(sa, d.U, s));
  SSA_TRY(ssa::launch_sample(sa, d.U, s));
  return SSA_OK;
}

int ssa_attend(const ssa_params* p, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens, const int32_t* sel_idx,
               const float* sel_logw, const int32_t* sel_count, void* out, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!p || p->key_layout != SSA_KEYS_WHOLE) return SSA_ERR_INVALID;
  return attend_impl(p, q, Keys{k_cache, nullptr}, v_cache, block_table, seq_lens, sel_idx,
                     sel_logw, sel_count, out, workspace, workspace_bytes, stream);
}

int ssa_attend_split(const ssa_params* p, const void* q, const void* k_dom, const void* k_rest,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* sel_idx, const float* sel_logw, const int32_t* sel_count,
                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!params_ok(p) || !split_keys_ok(p, k_dom, k_rest)) return SSA_ERR_INVALID;
  return attend_impl(p, q, Keys{k_dom, rest_of(p, k_rest)}, v_cache, block_table, seq_lens,
                     sel_idx, sel_logw, sel_count, out, workspace, workspace_bytes, stream);
}

int ssa_append_kv(const ssa_params* p, int32_t num_tokens, const void* k_new, const void* v_new,
                  const int32_t* block_table, const int32_t* seq_lens, void* k_cache,
                  void* k_rest, void* v_cache, void* stream) {
  if (!params_ok(p) || num_tokens < 0) return SSA_ERR_INVALID;
  if (!k_new || !v_new || !block_table || !seq_lens || !k_cache || !v_cache)
    return SSA_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return SSA_ERR_INVALID;
  if (p->key_layout == SSA_KEYS_WHOLE) {
    if (k_rest) return SSA_ERR_INVALID;
  } else if (!split_keys_ok(p, k_cache, k_rest)) {
    return SSA_ERR_INVALID;
  }
  if ((int64_t)p->num_kv_heads * p->head_dim > 8192) return SSA_ERR_INVALID;
  const int64_t ntok = (int64_t)p->batch * num_tokens;
  if (ntok == 0) return SSA_OK;
  if (ntok > INT32_MAX) return SSA_ERR_INVALID;
  ssa::AppendArgs a;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.k_rest = p->key_layout == SSA_KEYS_SPLIT
                 ? static_cast<uint16_t*>(const_cast<void*>(rest_of(p, k_rest)))
                 : nullptr;
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.B = p->batch;
  a.T = num_tokens;
  a.Hkv = p->num_kv_heads;
  a.d = p->head_dim;
  a.pair_begin = p->pair_begin;
  a.pair_count = p->pair_count;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.max_seq_len = p->max_seq_len;
  SSA_TRY(ssa::launch_append(a, static_cast<hipStream_t>(stream)));
  return SSA_OK;
}

int ssa_host_device_address(const void* host_ptr, void** dev_ptr) {
  if (!host_ptr || !dev_ptr) return SSA_ERR_INVALID;
  *dev_ptr = nullptr;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host_ptr), 0) != hipSuccess || !d) {
    (void)hipGetLastError();  // leave no sticky error for the next call
    return SSA_ERR_INVALID;
  }
  *dev_ptr = d;
  return SSA_OK;
}

int ssa_debug_philox(uint64_t seed, int32_t b, int32_t h, int32_t group, int32_t j0, int32_t n,
                     uint32_t* words, void* stream) {
  if (!words || n < 0 || j0 < 0 || b < 0 || h < 0 || group < 0) return SSA_ERR_INVALID;
  if ((int64_t)j0 + n > INT32_MAX) return SSA_ERR_INVALID;
  if (n == 0) return SSA_OK;
  SSA_TRY(ssa::launch_debug_philox(seed, b, h, group, j0, n, words,
                                   static_cast<hipStream_t>(stream)));
  return SSA_OK;
}

int ssa_debug_sexp(const float* x, float* y, int32_t n, void* stream) {
  if (!x || !y || n < 0) return SSA_ERR_INVALID;
  if (n == 0) return SSA_OK;
  SSA_TRY(ssa::launch_debug_sexp(x, y, n, static_cast<hipStream_t>(stream)));
  return SSA_OK;
}

int ssa_debug_tail_exp(const float* x, float* y, int32_t n, void* stream) {
  if (!x || !y || n < 0) return SSA_ERR_INVALID;
  if (n == 0) return SSA_OK;
  SSA_TRY(ssa::launch_debug_tail_exp(x, y, n, static_cast<hipStream_t>(stream)));
  return SSA_OK;
}

const char* ssa_error_string(int code) {
  switch (code) {
    case SSA_OK: return "ok";
    case SSA_ERR_INVALID: return "invalid argument";
    case SSA_ERR_WORKSPACE: return "workspace too small";
    case SSA_ERR_HIP: return "HIP launch or runtime error";
    case SSA_ERR_STATIC_LIMIT: return "step needs more than the static workspace (SSA_STATIC_WORKSPACE_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"

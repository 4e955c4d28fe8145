// Host-only driver for the C ABI's argument checks and workspace sizing,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// side.  The kernel launchers are stubs: every call made here must be turned
// away by the checks before any launch, and a stub that is reached is a
// failure.  Prints "ok" and exits 0 when every check holds.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "ssa.h"
#include "ssa_launch.h"

static int g_launches = 0;

namespace ssa {
int indexer_resident_workgroups(int) { return 0; }
hipError_t launch_init(uint32_t*, uint32_t*, uint32_t*, unsigned long long*, unsigned long long*,
                       int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_indexer(const IndexArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_score_hist(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_mass(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_threshold(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_filter(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_resolve(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_stop(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_sample(const SelectArgs&, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_attend(const AttendArgs&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_attend_select(const AttendArgs&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_append(const AppendArgs&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_merge(const AttendArgs&, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_refine(const RefineArgs&, int, int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_debug_philox(uint64_t, int, int, int, int, int, uint32_t*, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_debug_sexp(const float*, float*, int, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_debug_tail_exp(const float*, float*, int, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
}  // namespace ssa

static int g_failures = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::printf("check failed at line %d: %s\n", __LINE__, #cond);    \
      ++g_failures;                                                     \
    }                                                                   \
  } while (0)

static ssa_params valid() {
  ssa_params p{};
  p.batch = 2;
  p.num_q_heads = 32;
  p.num_kv_heads = 8;
  p.head_dim = 128;
  p.block_size = SSA_BLOCK_TOKENS;
  p.max_blocks_per_seq = 64;
  p.num_blocks = 128;
  p.max_seq_len = 1000;
  p.pair_begin = 32;
  p.pair_count = 32;
  p.num_splits = 0;
  p.out_dtype = SSA_F32;
  p.softmax_scale = 0.0f;
  p.num_queries = 1;
  p.query_group = 1;
  p.early_stop = 0.0f;
  p.key_layout = SSA_KEYS_WHOLE;
  p.max_topk = 0;
  return p;
}

int main() {
  // Workspace sizing over ordinary and extreme parameters: a size or 0,
  // never an overflowed size (UBSan reports signed overflow).
  {
    const ssa_params p = valid();
    CHECK(ssa_workspace_bytes(&p) > 0);
    CHECK(ssa_num_chunks(&p) == 1);
    CHECK(ssa_workspace_bytes(nullptr) == 0);
    const int32_t batches[] = {1, 7, 1 << 10, 1 << 20, INT_MAX};
    const int32_t lens[] = {1, 4095, 4097, 1 << 20, SSA_MAX_SEQ_LEN, SSA_MAX_SEQ_LEN + 1};
    const int32_t kvs[] = {1, 8, 1 << 12, INT_MAX};
    const int32_t tq[] = {1, 4, 1 << 16, INT_MAX};
    for (int32_t b : batches)
      for (int32_t L : lens)
        for (int32_t hkv : kvs)
          for (int32_t T : tq) {
            ssa_params q = valid();
            q.batch = b;
            q.max_seq_len = L;
            q.max_blocks_per_seq = L > 0 ? (L + 15) / 16 : 1;
            q.num_kv_heads = hkv;
            q.num_q_heads = hkv <= INT_MAX / 4 ? 4 * hkv : hkv;
            q.num_queries = T;
            q.query_group = T;
            (void)ssa_workspace_bytes(&q);
            (void)ssa_num_chunks(&q);
          }
  }
  // Every entry point turns away a null params pointer and bad arguments.
  std::vector<unsigned char> ws_small(64);
  alignas(16) static unsigned char buf[1 << 16];
  void* dev = buf;
  const int32_t* i32 = reinterpret_cast<const int32_t*>(buf);
  const uint64_t* u64 = reinterpret_cast<const uint64_t*>(buf);
  const float* f32 = reinterpret_cast<const float*>(buf);
  {
    CHECK(ssa_decode(nullptr, dev, dev, dev, i32, i32, i32, nullptr, i32, u64, dev, dev, 1 << 16,
                     nullptr) != SSA_OK);
    const ssa_params p = valid();
    // workspace too small
    CHECK(ssa_decode(&p, dev, dev, dev, i32, i32, i32, nullptr, i32, u64, dev, ws_small.data(),
                     ws_small.size(), nullptr) != SSA_OK);
    // null and misaligned buffers
    const size_t need = ssa_workspace_bytes(&p);
    std::vector<unsigned char> ws(need + 256);
    void* w = ws.data();
    CHECK(ssa_decode(&p, nullptr, dev, dev, i32, i32, i32, nullptr, i32, u64, dev, w, need,
                     nullptr) != SSA_OK);
    CHECK(ssa_decode(&p, buf + 2, dev, dev, i32, i32, i32, nullptr, i32, u64, dev, w, need,
                     nullptr) != SSA_OK);
    CHECK(ssa_score(&p, dev, dev, i32, i32, nullptr, w, need, nullptr) != SSA_OK);
    CHECK(ssa_select(&p, nullptr, i32, i32, nullptr, i32, u64, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, w, need,
                     nullptr) != SSA_OK);
    // refine mode: not with early stopping, the staged query slices must fit,
    // and the selection needs the query and keys
    {
      ssa_params rp = valid();
      rp.num_queries = 4;
      rp.query_group = 4;
      rp.refine = 2;
      CHECK(ssa_workspace_bytes(&rp) > ssa_workspace_bytes(&p));
      rp.refine = -1;
      CHECK(ssa_workspace_bytes(&rp) == 0);
      rp.refine = 2;
      rp.early_stop = 0.5f;
      CHECK(ssa_workspace_bytes(&rp) == 0);
      rp.early_stop = 0.0f;
      rp.num_queries = 64;
      rp.query_group = 64;  // 64 members x 4 heads x 64 scored dims > 8192 staged floats
      CHECK(ssa_workspace_bytes(&rp) == 0);
      rp.num_queries = 4;
      rp.query_group = 4;
      const size_t need_r = ssa_workspace_bytes(&rp);
      std::vector<unsigned char> wr(need_r + 256);
      float* sc = reinterpret_cast<float*>(buf);
      int32_t* o32 = reinterpret_cast<int32_t*>(buf);
      float* of = reinterpret_cast<float*>(buf);
      CHECK(ssa_select(&rp, sc, i32, i32, nullptr, i32, u64, nullptr, nullptr, dev, nullptr, i32,
                       o32, of, o32, of, wr.data(), need_r, nullptr) == SSA_ERR_INVALID);
      CHECK(ssa_select(&rp, sc, i32, i32, f32, i32, u64, nullptr, dev, dev, nullptr, i32, o32,
                       of, o32, of, wr.data(), need_r, nullptr) == SSA_ERR_INVALID);
      CHECK(ssa_decode(&rp, dev, dev, dev, i32, i32, i32, f32, i32, u64, dev, wr.data(), need_r,
                       nullptr) == SSA_ERR_INVALID);
    }
    // early stopping: the stratum bound and the rows must fit its kernels, and
    // the selection needs the query and keys
    {
      ssa_params es = valid();
      es.early_stop = 0.1f;
      CHECK(ssa_workspace_bytes(&es) > 0);  // max_seq_len 1000 bounds the stratum
      es.max_seq_len = 16385;
      es.max_blocks_per_seq = 1025;
      CHECK(ssa_workspace_bytes(&es) == 0);
      es.max_topk = SSA_STOP_MAX_STRATUM;
      CHECK(ssa_workspace_bytes(&es) > 0);
      es.max_topk = -1;
      CHECK(ssa_workspace_bytes(&es) == 0);
      es.max_topk = 100;
      es.num_queries = 8;
      es.query_group = 8;  // 8 members x 4 heads > SSA_STOP_MAX_ROWS
      CHECK(ssa_workspace_bytes(&es) == 0);
      es.query_group = 4;
      const size_t need_es = ssa_workspace_bytes(&es);
      CHECK(need_es > 0);
      std::vector<unsigned char> wes(need_es + 256);
      float* sc = reinterpret_cast<float*>(buf);
      int32_t* o32 = reinterpret_cast<int32_t*>(buf);
      float* of = reinterpret_cast<float*>(buf);
      CHECK(ssa_select(&es, sc, i32, i32, nullptr, i32, u64, nullptr, nullptr, dev, nullptr, i32,
                       o32, of, o32, of, wes.data(), need_es, nullptr) == SSA_ERR_INVALID);
      CHECK(ssa_select(&es, sc, i32, i32, nullptr, i32, u64, nullptr, dev, nullptr, nullptr, i32,
                       o32, of, o32, of, wes.data(), need_es, nullptr) == SSA_ERR_INVALID);
      CHECK(ssa_select(&es, sc, i32, i32, nullptr, i32, u64, nullptr, dev, dev, nullptr, nullptr,
                       o32, of, o32, of, wes.data(), need_es, nullptr) == SSA_ERR_INVALID);
    }
    CHECK(ssa_attend(&p, dev, dev, dev, i32, i32, nullptr, f32, i32, dev, w, need, nullptr) !=
          SSA_OK);
    // split-key entry points reject whole-key params, and the reverse
    CHECK(ssa_decode_split(&p, dev, dev, dev, dev, i32, i32, i32, nullptr, i32, u64, dev, w,
                           need, nullptr, nullptr) != SSA_OK);
    CHECK(ssa_attend_split(&p, dev, dev, dev, dev, i32, i32, i32, f32, i32, dev, w, need,
                           nullptr) != SSA_OK);
    ssa_params sp = valid();
    sp.key_layout = SSA_KEYS_SPLIT;
    CHECK(ssa_attend(&sp, dev, dev, dev, i32, i32, i32, f32, i32, dev, w, need, nullptr) !=
          SSA_OK);
    sp.key_layout = 7;
    CHECK(ssa_workspace_bytes(&sp) == 0);
    // append: bad token count, null buffers, too many heads x dims
    CHECK(ssa_append_kv(&p, -1, dev, dev, i32, i32, dev, nullptr, dev, nullptr) != SSA_OK);
    CHECK(ssa_append_kv(&p, 1, nullptr, dev, i32, i32, dev, nullptr, dev, nullptr) != SSA_OK);
    CHECK(ssa_append_kv(&p, 1, dev, dev, i32, i32, dev, dev, dev, nullptr) != SSA_OK);
    ssa_params wide = valid();
    wide.num_kv_heads = 128;
    wide.num_q_heads = 128;
    CHECK(ssa_append_kv(&wide, 1, dev, dev, i32, i32, dev, nullptr, dev, nullptr) != SSA_OK);
    // invalid parameter values
    ssa_params bad = valid();
    bad.head_dim = 96;
    CHECK(ssa_workspace_bytes(&bad) == 0);
    bad = valid();
    bad.num_q_heads = 30;
    CHECK(ssa_workspace_bytes(&bad) == 0);
    bad = valid();
    bad.pair_count = 12;
    CHECK(ssa_workspace_bytes(&bad) == 0);
    bad = valid();
    bad.max_seq_len = 0;
    CHECK(ssa_workspace_bytes(&bad) == 0);
    bad = valid();
    bad.num_splits = -1;
    CHECK(ssa_workspace_bytes(&bad) == 0);
    bad = valid();
    bad.query_group = 0;
    CHECK(ssa_workspace_bytes(&bad) == 0);
    // debug hooks
    CHECK(ssa_debug_philox(0, 0, 0, 0, 0, 4, nullptr, nullptr) != SSA_OK);
    CHECK(ssa_debug_sexp(nullptr, nullptr, 4, nullptr) != SSA_OK);
    // error strings for known and unknown codes
    for (int code = -20; code <= 2; ++code) CHECK(ssa_error_string(code) != nullptr);
  }
  CHECK(g_launches == 0);
  if (g_failures == 0) std::printf("ok\n");
  return g_failures == 0 ? 0 : 1;
}

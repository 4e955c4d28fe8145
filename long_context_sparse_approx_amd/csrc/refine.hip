// Refine mode of query groups: every member re-ranks the group's candidate
// list with its own query.
//
// "PIVOT slashes sparse-attention indexer cost", "The two observations behind
// PIVOT" (a group of consecutive queries is scored once through its mean, and
// the proxy's candidate list is refined for each member) and "Two operating
// modes" (refine keeps the dense indexer's accuracy).  The group's selection
// has already run with a deterministic stratum of r * k tokens: that stratum
// is the candidate list C, and the group's tail sample R_C was drawn with
// the normaliser W_C of the group's span minus C.  Then, per member t:
//   refine_score:  its own score of every candidate (its G heads' partial
//                  logits over the scored pairs), in a specified float32
//                  order: per head, each 8-dim slice summed in dim order and
//                  the slices pairwise (a butterfly over the lanes holding a
//                  token's 16-byte slices), the heads summed in head order,
//                  times fl32(fl32(scale) / G);
//   refine_select: its stratum S_t = the k_t candidates inside its span first
//                  in the order (own score descending, position ascending),
//                  found by a radix select over 56-bit words
//                  ((~own key) << 24) | position, and its normaliser
//                  W_t = W_C + the proxy weight of the candidates it drops
//                  (float64, fixed order), both sums direct;
//   refine_emit:   its selection segment per chunk: S_t, then the samples:
//                  dropped candidates and the group's samples inside its span
//                  that pass fl(u_j W_t) < fl(m w_j) with the group's
//                  uniforms and the proxy's weights.  W_t >= W_C, so the
//                  group's sample holds every token outside C that the member
//                  can draw.
// Every decision is integer or float32 in a fixed order: bitwise
// reproducible, no floating-point atomics.
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

constexpr int kRS = 256;     // threads of a score or emit workgroup
constexpr int kRT = 1024;    // threads of a member's select workgroup (one per member unit)
constexpr int kRefineQ = 8192;  // floats of the group's staged query slices

__device__ __forceinline__ void decode_member(const RefineArgs& a, int v, int* b, int* t, int* h,
                                              int* u) {
  *h = v % a.Hkv;
  const int bt = v / a.Hkv;
  *t = bt % a.T;
  *b = bt / a.T;
  *u = (*b * a.NG + *t / a.g) * a.Hkv + *h;
}

__device__ __forceinline__ unsigned long long member_word(uint32_t own_key, int pos) {
  return ((unsigned long long)(~own_key) << 24) | (uint32_t)pos;
}

// Grid: (chunks, group units) x kRS threads; dynamic LDS holds the group's
// scored query slices (nmem * G * 2 * pair_count floats).  LPT lanes per
// candidate (one 16-byte slice of its scored dims each); all the group's
// members are scored from one load of the slice.  A thread's candidates
// (kPass passes of kRS / LPT) have their positions, then block ids and proxy
// scores, then slices loaded in three rounds, each round's loads all in
// flight together.  Each candidate's proxy weight sexp(s - M) is stored
// beside the group's entry, so the member selections read it in order
// instead of gathering scores.
constexpr int kPass = 4;
template <int LPT>
__global__ __launch_bounds__(kRS) void refine_score_kernel(RefineArgs a) {
  extern __shared__ float qsh[];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int c0 = c * kChunk;
  if (c0 >= ui.L) return;  // uniform
  const size_t ci = (size_t)u * a.nchunk + c;
  const int n_det = clamp_count(a.gsel_cnt[2 * ci], kChunk);
  if (n_det == 0) return;  // uniform
  const int b = ui.b, h = ui.h;
  const int t0 = ui.grp * a.g;
  const int nmem = min(a.g, a.T - t0);
  const int nd = 2 * a.pair_count;
  const int rowq = a.G * nd;  // floats per member
  for (int i = threadIdx.x; i < nmem * rowq; i += kRS) {
    const int mi = i / rowq;
    const int r = i - mi * rowq;
    const int gh = r / nd;
    const int e = r - gh * nd;
    const uint16_t bits =
        a.q[((size_t)(b * a.T + t0 + mi) * a.Hq + h * a.G + gh) * a.d + 2 * a.pair_begin + e];
    qsh[i] = __uint_as_float((uint32_t)bits << 16);
  }
  const int sl = threadIdx.x % LPT;
  const int tk = threadIdx.x / LPT;
  constexpr int TPP = kRS / LPT;  // candidates per pass
  const int32_t* pidx = a.gsel_idx + (size_t)u * a.seg_ld + c0;
  const int* btrow = a.block_table + (size_t)b * a.max_blocks;
  const float* srow = a.scores + (size_t)u * a.score_ld;
  float* pw = a.cand_pw + (size_t)u * a.seg_ld + c0;
  const float M = reinterpret_cast<const UnitState*>(a.gstate)[u].M;
  __syncthreads();
  for (int base = 0; base < n_det; base += kPass * TPP) {  // uniform trip count
    int pos[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int i = base + p * TPP + tk;
      pos[p] = i < n_det ? min(max(pidx[i], 0), ui.L - 1) : 0;
    }
    int blk[kPass];
    float ps[kPass];  // the candidate's proxy score
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      blk[p] = btrow[pos[p] >> 4];
      ps[p] = srow[pos[p]];
    }
    uint4 kv[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int bk = blk[p] < 0 ? 0 : (blk[p] >= a.num_blocks ? a.num_blocks - 1 : blk[p]);
      const size_t row = (size_t)(bk * a.Hkv + h) * kBlockTokens + (pos[p] & 15);
      kv[p] = *reinterpret_cast<const uint4*>(a.k_cache + row * a.key_ld + a.key_off + sl * 8);
    }
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int i = base + p * TPP + tk;
      if (base + p * TPP >= n_det) break;  // uniform
      if (i < n_det && sl == 0) pw[i] = sexp(ps[p] - M);
      const float kf[8] = {bf16_lo(kv[p].x), bf16_hi(kv[p].x), bf16_lo(kv[p].y),
                           bf16_hi(kv[p].y), bf16_lo(kv[p].z), bf16_hi(kv[p].z),
                           bf16_lo(kv[p].w), bf16_hi(kv[p].w)};
      for (int mi = 0; mi < nmem; ++mi) {  // uniform
        float acc = 0.0f;
        for (int gh = 0; gh < a.G; ++gh) {  // uniform
          const float* qs = qsh + mi * rowq + gh * nd + sl * 8;
          float d = qs[0] * kf[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) d = d + qs[e] * kf[e];  // exact products, dim order
          d = butterfly<LPT>(d);
          acc = gh == 0 ? d : acc + d;
        }
        const float s = acc * a.own_scale;
        if (i < n_det && sl == 0) {
          const int v = (b * a.T + t0 + mi) * a.Hkv + h;
          a.own_key[(size_t)v * a.seg_ld + c0 + i] = order_key(s);
        }
      }
    }
  }
}

// The first bin (from bin 0 up) where the running count reaches k >= 1, and
// the remainder; every thread of the block calls; kRT threads, nbins a
// multiple of kRT.
__device__ __forceinline__ void find_bin_up(const uint32_t* hist, int nbins, int k, int* scan,
                                            int* pair, int* bin_out, int* rem_out) {
  const int per = nbins / kRT;
  const int lo = threadIdx.x * per;
  int mine = 0;
  for (int i = 0; i < per; ++i) mine += (int)hist[lo + i];
  int total;
  const int before = block_exclusive_scan<kRT>(mine, scan, &total);
  if (before < k && k <= before + mine) {
    int run = before;
    for (int i = 0; i < per; ++i) {
      const int cnt = (int)hist[lo + i];
      if (run + cnt >= k) {
        pair[0] = lo + i;
        pair[1] = k - run;
        break;
      }
      run += cnt;
    }
  }
  __syncthreads();
  *bin_out = pair[0];
  *rem_out = pair[1];
  __syncthreads();
}

// Grid: member units x kRT threads.  The group's candidates are flattened
// over its chunks (a prefix of the chunks' counts in LDS) and thread t takes
// items t, t + kRT, ...: the first kKeep of them are read once into
// registers as words, so the radix passes touch only registers and LDS (a
// thread's further items, when the list exceeds kRT * kKeep, are read again
// on every pass).
constexpr int kKeep = 24;
constexpr int kMaxChunks = SSA_MAX_SEQ_LEN / SSA_CHUNK_TOKENS;
constexpr int kChunkTab = 4096;  // item-to-chunk table entries (groups of <= 2^18 candidates)
__global__ __launch_bounds__(kRT) void refine_select_kernel(RefineArgs a) {
  constexpr int kDig = 8192;
  __shared__ uint32_t hist[kDig];
  __shared__ int cpre[kMaxChunks + 1];  // candidates in chunks before c
  __shared__ int ctab[kChunkTab];  // chunk of item 64 m
  __shared__ int scan[kRT / 64];
  __shared__ int pair[2];
  __shared__ double dscr[kRT / 64];
  const int v = blockIdx.x;
  int b, t, h, u;
  decode_member(a, v, &b, &t, &h, &u);
  const UnitState gs = reinterpret_cast<const UnitState*>(a.gstate)[u];
  const double gw = a.gw64[u];
  const int P = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int Lt = member_span(P, a.T, t);
  const int Lg = gs.L;
  const int k = min(max(a.topk[b], 0), a.max_topk);
  const int m = max(a.sample_budget[b], 0);
  const int nc = (Lg + kChunk - 1) / kChunk;
  const size_t cu = (size_t)u * a.nchunk;
  const int32_t* gidx = a.gsel_idx + (size_t)u * a.seg_ld;
  const uint32_t* okey = a.own_key + (size_t)v * a.seg_ld;
  const float* gpw = a.cand_pw + (size_t)u * a.seg_ld;
  if (threadIdx.x < 2) hist[threadIdx.x] = 0u;
  // Prefix of the chunks' candidate counts.
  {
    int run = 0;
    for (int c0 = 0; c0 < nc; c0 += kRT) {
      const int c = c0 + threadIdx.x;
      const int n = c < nc ? clamp_count(a.gsel_cnt[2 * (cu + c)], kChunk) : 0;
      int tot;
      const int ex = block_exclusive_scan<kRT>(n, scan, &tot);
      if (c < nc) cpre[c] = run + ex;
      run += tot;
    }
    if (threadIdx.x == 0) cpre[nc] = run;
    __syncthreads();
  }
  const int N = cpre[nc];
  // The chunk of every 64th item (a chunk holds ~80 at 50x sparsity, so an
  // item's chunk is that entry's or one of the next few); groups too large
  // for the table search the prefix instead.
  const bool tab = N <= kChunkTab * 64;  // uniform
  if (tab) {
    for (int c = threadIdx.x; c < nc; c += kRT) {
      const int first = (cpre[c] + 63) >> 6, end = (cpre[c + 1] + 63) >> 6;
      for (int m = first; m < end; ++m) ctab[m] = c;
    }
    __syncthreads();
  }
  // Item j's place in the group's segments.
  auto at_of = [&](int j) -> int {  // < nchunk * 4096 <= 2^24
    int c;
    if (tab) {
      c = ctab[j >> 6];  // cpre[c] <= 64 (j >> 6) <= j
      while (cpre[c + 1] <= j) ++c;
    } else {
      int lo = 0, hi = nc;  // cpre[lo] <= j < cpre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cpre[mid] <= j) lo = mid; else hi = mid;
      }
      c = lo;
    }
    return c * kChunk + (j - cpre[c]);
  };
  auto word_of = [&](int j) -> unsigned long long {
    const int at = at_of(j);
    return member_word(okey[at], min(max(gidx[at], 0), max(Lg - 1, 0)));
  };
  unsigned long long wv[kKeep];
  {
    int at[kKeep];
#pragma unroll
    for (int e = 0; e < kKeep; ++e) {
      const int j = threadIdx.x + e * kRT;
      at[e] = j < N ? at_of(j) : 0;
    }
#pragma unroll
    for (int e = 0; e < kKeep; ++e) {  // every load of the thread's items in flight
      const int j = threadIdx.x + e * kRT;
      wv[e] = j < N ? member_word(okey[at[e]], min(max(gidx[at[e]], 0), max(Lg - 1, 0))) : ~0ull;
    }
  }
  // Every item of this thread (registers first, then memory), with f(word).
  auto each = [&](auto&& f) {
#pragma unroll
    for (int e = 0; e < kKeep; ++e)
      if (threadIdx.x + e * kRT < N) f(wv[e]);
    for (int j = threadIdx.x + kKeep * kRT; j < N; j += kRT) f(word_of(j));
  };
  auto pos_of = [](unsigned long long w) { return (int)(w & 0xffffffull); };
  int ncand = 0;
  each([&](unsigned long long w) { ncand += pos_of(w) < Lt ? 1 : 0; });
  ncand = block_sum_i32<kRT>(ncand, scan);
  const int kt = min(k, ncand);
  int flags = 0;
  if (Lt == 0 || (gs.flags & kFlagEmpty)) flags |= kFlagEmpty;
  else if ((int64_t)kt + m >= (int64_t)Lt) flags |= kFlagDense;
  unsigned long long vstar = 0ull;
  double W = 0.0;
  if (!(flags & (kFlagEmpty | kFlagDense))) {
    if (kt > 0) {
      // Radix select of the kt-th smallest word.  The candidates' inverted
      // keys span [lo, lo + 2^kb), so the word's key part is taken relative
      // to lo: 12-bit digits then cover the part of the key that differs
      // (the top bits of the order key, sign and exponent, are shared by
      // most candidates and would send them all to a few bins).
      uint32_t lo = 0xffffffffu, hi = 0u;
      each([&](unsigned long long w) {
        if (pos_of(w) < Lt) {
          const uint32_t ik = (uint32_t)(w >> 24);
          lo = ik < lo ? ik : lo;
          hi = ik > hi ? ik : hi;
        }
      });
      lo = ~wave_max_u32(~lo);
      hi = wave_max_u32(hi);
      if ((threadIdx.x & 63) == 0) {
        atomicMax(&hist[0], ~lo);  // hist[0..1] as scratch: both start at 0
        atomicMax(&hist[1], hi);
      }
      __syncthreads();
      lo = ~hist[0];
      const int kb = 32 - __builtin_clz((hist[1] - lo) | 1u);  // bits of the key part
      __syncthreads();
      const int nbits = kb + 24;
      auto rel = [&](unsigned long long w) {
        return ((unsigned long long)((uint32_t)(w >> 24) - lo) << 24) | (w & 0xffffffull);
      };
      unsigned long long prefix = 0ull;
      int rank = kt;
      // Digits of at most 13 bits, the key part split evenly (two passes for
      // the usual range of up to 26 bits); then the position's two 12-bit
      // digits, only when the candidates tied on the threshold key are not
      // all taken.
      const int kpass = (kb + 12) / 13;
      int top = nbits;
      for (int d = 0; d < kpass + 2; ++d) {
        const int key_bits_left = top - 24;
        const int wd = d < kpass ? (key_bits_left + (kpass - d) - 1) / (kpass - d) : 12;
        const int sh = top - wd;
        for (int i = threadIdx.x; i < kDig; i += kRT) hist[i] = 0u;
        __syncthreads();
        each([&](unsigned long long w) {
          const unsigned long long r = rel(w);
          if (pos_of(w) < Lt && (r >> top) == prefix)
            atomicAdd(&hist[(r >> sh) & ((1u << wd) - 1u)], 1u);
        });
        __syncthreads();
        int bin, rem;
        find_bin_up(hist, kDig, rank, scan, pair, &bin, &rem);
        const bool whole = hist[bin] == (uint32_t)rem;  // every tie on the key taken
        __syncthreads();
        prefix = (prefix << wd) | (unsigned long long)bin;
        rank = rem;
        top = sh;
        if (top == 24 && whole) {  // the key part is resolved and its ties all fit
          prefix = (prefix << 24) | 0xffffffull;
          top = 0;
          break;
        }
      }
      // back to the absolute word
      vstar = ((unsigned long long)((uint32_t)(prefix >> 24) + lo) << 24) | (prefix & 0xffffffull);
    }
    // W_t: the group's tail sum plus the proxy weight of every candidate the
    // member does not keep (those outside its span included).  The weights
    // were stored by the score kernel beside the entries: one round of loads
    // in order.
    double ws = 0.0;
    float pwv[kKeep];
#pragma unroll
    for (int e = 0; e < kKeep; ++e) {
      const int j = threadIdx.x + e * kRT;
      pwv[e] = j < N ? gpw[at_of(j)] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kKeep; ++e) {
      const unsigned long long w = wv[e];
      const bool kept = kt > 0 && pos_of(w) < Lt && w <= vstar;
      if (threadIdx.x + e * kRT < N && !kept) ws += (double)pwv[e];
    }
    for (int j = threadIdx.x + kKeep * kRT; j < N; j += kRT) {
      const int at = at_of(j);
      const unsigned long long w = member_word(okey[at], min(max(gidx[at], 0), max(Lg - 1, 0)));
      const bool kept = kt > 0 && pos_of(w) < Lt && w <= vstar;
      if (!kept) ws += (double)gpw[at];
    }
    W = gw + block_sum_f64<kRT>(ws, dscr);
  }
  const float Wt = a.w_in ? a.w_in[v] : (float)W;
  if (!(flags & (kFlagEmpty | kFlagDense)) && m > 0 && Lg - kt > 0 && Wt > 0.0f)
    flags |= kFlagSample;
  if (kt == 0) flags |= kFlagNoTopk;
  if (threadIdx.x == 0) {
    MemberState ms;
    ms.vstar = vstar;
    ms.W = (flags & (kFlagEmpty | kFlagDense)) ? 0.0f : Wt;
    ms.M = gs.M;
    ms.k = kt;
    ms.flags = flags;
    ms.L = Lt;
    ms.m = m;
    reinterpret_cast<MemberState*>(a.mstate)[v] = ms;
    if (a.norm_out) {
      a.norm_out[2 * (size_t)v] = gs.M;
      a.norm_out[2 * (size_t)v + 1] = ms.W;
    }
  }
}

constexpr uint32_t kMarkNone = 0xffffffffu;
constexpr uint32_t kMarkDet = 0xfffffffeu;

// Grid: (chunks, group units) x kRS threads.  The chunk's group entries
// (candidates, then the group's samples), their proxy weights and uniforms
// are loaded and drawn once; then each member in turn marks its stratum and
// samples in an LDS map of the chunk and writes its segment from it.
__global__ __launch_bounds__(kRS) __attribute__((amdgpu_waves_per_eu(8))) void refine_emit_kernel(RefineArgs a) {
  __shared__ uint32_t mark[kChunk];
  __shared__ int scan_scr[kRS / 64];
  constexpr int kPerT = kChunk / kRS;  // 16: also the most group entries per thread
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b, h = ui.h;
  const int t0 = ui.grp * a.g;
  const int nmem = min(a.g, a.T - t0);
  const int c0 = c * kChunk;
  const size_t ci = (size_t)u * a.nchunk + c;
  const int n_det = c0 < ui.L ? clamp_count(a.gsel_cnt[2 * ci], kChunk) : 0;
  const int n_smp = c0 < ui.L ? clamp_count(a.gsel_cnt[2 * ci + 1], kChunk - n_det) : 0;
  const int n_all = n_det + n_smp;
  const int32_t* gidx = a.gsel_idx + (size_t)u * a.seg_ld + c0;
  const float* srow = a.scores + (size_t)u * a.score_ld;
  const float M = reinterpret_cast<const UnitState*>(a.gstate)[u].M;
  const uint64_t seed = a.seed[b];
  // Entry i's position (-1 outside the chunk or span), proxy weight and
  // uniform.  A thread keeps its first kFast entries (i = threadIdx.x +
  // e * kRS) in registers; a chunk rarely holds more than kRS * kFast
  // entries, and further ones are computed again for every member.
  constexpr int kFast = 2;
  // A candidate's weight was stored by the score kernel; a sample's is
  // computed here.
  const float* cpw = a.cand_pw + (size_t)u * a.seg_ld + c0;
  auto entry = [&](int i, int& p, float& w, float& un) {
    p = i < n_all ? gidx[i] : -1;
    const bool in = (unsigned)(p - c0) < (unsigned)kChunk && p < ui.L;
    if (!in) p = -1;
    w = !in ? 0.0f : (i < n_det ? cpw[i] : sexp(srow[p] - M));
    un = 0.0f;
    if (in) {
      const uint4 wd = philox_block(seed, b, h, (uint32_t)p >> 2, ui.grp);
      const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
      un = uniform24(words[p & 3]);
    }
  };
  int pos[kFast];
  float wgt[kFast], uni[kFast];
#pragma unroll
  for (int e = 0; e < kFast; ++e) entry(threadIdx.x + e * kRS, pos[e], wgt[e], uni[e]);
  for (int mi = 0; mi < nmem; ++mi) {  // uniform
    const int v = (b * a.T + t0 + mi) * a.Hkv + h;
    const MemberState ms = reinterpret_cast<const MemberState*>(a.mstate)[v];
    int32_t* cnt = a.msel_cnt + ((size_t)v * a.nchunk + c) * 2;
    if (c0 >= ms.L || (ms.flags & kFlagEmpty)) {  // uniform
      if (threadIdx.x == 0) {
        cnt[0] = 0;
        cnt[1] = 0;
      }
      continue;
    }
    const int nvalid = min(kChunk, ms.L - c0);
    const bool dense = ms.flags & kFlagDense;
    const bool sampling = ms.flags & kFlagSample;
    const bool notopk = ms.flags & kFlagNoTopk;
    const uint32_t* okey = a.own_key + (size_t)v * a.seg_ld + c0;
    uint32_t ok[kFast];
#pragma unroll
    for (int e = 0; e < kFast; ++e) {
      const int i = threadIdx.x + e * kRS;
      ok[e] = (!dense && i < n_det) ? okey[i] : 0u;
    }
    __syncthreads();  // the previous member's map has been read
    for (int i = threadIdx.x; i < kChunk; i += kRS)
      mark[i] = (dense && i < nvalid) ? kMarkDet : kMarkNone;
    __syncthreads();
    if (!dense) {
      const float mf = (float)ms.m;
      auto place = [&](int i, int p, float w, float un, uint32_t key) {
        if (p < 0 || p - c0 >= nvalid) return;  // not in the member's span
        if (i < n_det && !notopk && member_word(key, p) <= ms.vstar) {
          mark[p - c0] = kMarkDet;
        } else if (sampling) {
          const float mw = mf * w;
          if (un * ms.W < mw) mark[p - c0] = __float_as_uint(-logf(fminf(1.0f, mw / ms.W)));
        }
      };
#pragma unroll
      for (int e = 0; e < kFast; ++e)
        place(threadIdx.x + e * kRS, pos[e], wgt[e], uni[e], ok[e]);
      for (int i = threadIdx.x + kFast * kRS; i < n_all; i += kRS) {
        int p;
        float w, un;
        entry(i, p, w, un);
        place(i, p, w, un, i < n_det ? okey[i] : 0u);
      }
    }
    __syncthreads();
    // Compaction from the membership map (16 consecutive positions per thread).
    const int tb = threadIdx.x * kPerT;
    uint32_t smask = 0u, rmask = 0u;
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const uint32_t mk = mark[tb + i];
      smask |= (uint32_t)(mk == kMarkDet) << i;
      rmask |= (uint32_t)(mk < kMarkDet) << i;
    }
    int packed_tot;
    const int packed = block_exclusive_scan<kRS>(__popc(smask) | (__popc(rmask) << 16),
                                                 scan_scr, &packed_tot);
    const int totS = packed_tot & 0xffff;
    const int totR = packed_tot >> 16;
    int32_t* sidx = a.msel_idx + (size_t)v * a.seg_ld + c0;
    float* slw = a.msel_logw + (size_t)v * a.seg_ld + c0;
    int ws = packed & 0xffff, wr = totS + (packed >> 16);
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const uint32_t bit = 1u << i;
      if ((smask | rmask) & bit) {
        const int p = c0 + tb + i;
        if (smask & bit) {
          sidx[ws] = p;
          slw[ws] = 0.0f;
          ++ws;
        } else {
          sidx[wr] = p;
          slw[wr] = __uint_as_float(mark[tb + i]);
          ++wr;
        }
      }
    }
    if (threadIdx.x == 0) {
      cnt[0] = totS;
      cnt[1] = totR;
    }
  }
}

}  // namespace

hipError_t launch_refine(const RefineArgs& a, int group_units, int member_units,
                         hipStream_t stream) {
  const int nmem = a.g < a.T ? a.g : a.T;
  if (nmem * a.G * 2 * a.pair_count > kRefineQ) return hipErrorInvalidValue;
  const dim3 sg(a.nchunk, group_units);
  const size_t qbytes = (size_t)nmem * a.G * 2 * a.pair_count * sizeof(float);
  switch (a.pair_count / 4) {  // lanes per candidate: 2 * pair_count / 8
    case 1: refine_score_kernel<1><<<sg, kRS, qbytes, stream>>>(a); break;
    case 2: refine_score_kernel<2><<<sg, kRS, qbytes, stream>>>(a); break;
    case 4: refine_score_kernel<4><<<sg, kRS, qbytes, stream>>>(a); break;
    case 8: refine_score_kernel<8><<<sg, kRS, qbytes, stream>>>(a); break;
    case 16: refine_score_kernel<16><<<sg, kRS, qbytes, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  refine_select_kernel<<<member_units, kRT, 0, stream>>>(a);
  refine_emit_kernel<<<dim3(a.nchunk, group_units), kRS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ssa

// Stages 2-4: the deterministic stratum (exact top-k) and the Poisson tail
// sample of every (batch, kv head).
//
// "Stratified Sparse Attention speeds up decoding 2.96x at 1M context",
// sections "Where sparse attention loses quality" (top-k read
// deterministically) and "How SSA stratifies the cache" (the rest of the
// cache is sampled with probability proportional to an approximate attention
// estimate and corrected by the inclusion probability).
//
//   top-k:  the k tokens with the largest float32 score order keys, ties to
//           the lower index; found by a three-digit radix select (11/11/10
//           bits) whose first digit histogram comes from stage 1;
//   top-p:  optionally the stratum ends earlier, at the shortest prefix of
//           that order whose mass units floor(2^38 sexp(s_j - M)) reach
//           ceil(p * total); the same radix select runs on mass histograms
//           (64-bit integer sums) beside the count histograms, and at each
//           digit the bound reached first decides;
//   tail:   w_j = sexp(s_j - M), W = sum over the tail, computed directly in
//           fp64 (never as total minus top-k, which cancels);
//   sample: include j iff fl(u_j * W) < fl(m * w_j), u_j from Philox4x32-10
//           keyed by the sequence's seed with counter (j >> 2, h, b, group);
//           pi_j = min(1, fl(m * w_j) / W); the logit bias is -log(pi_j);
//   stop:   optionally the stratum is cut by the early-stopping rule (the
//           section of that name below).
//
// A sequence is processed in 4096-token chunks.  Each chunk's selected tokens
// are written to its own segment in index order, so no grid-wide ordering is
// needed and the attention stage splits work along chunk boundaries.  Every
// sum has a fixed order and only integer atomics are used: results are
// bitwise reproducible.
//
// Only one pass reads every score (the filter).  Besides the threshold-digit
// candidates and the tail weights it lists, per chunk, the tokens above the
// threshold digit and the tail tokens that pass a necessary inclusion test,
// fl(u_j * W_lb) < fl(m * w_j), with W_lb <= W a lower bound of the
// normaliser taken from the first-digit histogram (u_j * W_lb <= u_j * W and
// rounding is monotone, so no token that the exact test would include is
// dropped).  The final sample pass only visits these lists.
#include "select_device.h"
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

// ------------------------------------------------------------------ mass
// Top-p only.  Per chunk: every token's mass units go to the unit's
// first-digit mass histogram (integer atomics: the sums do not depend on the
// order of arrival).
__global__ __launch_bounds__(kNT) void mass_kernel(SelectArgs a) {
  __shared__ unsigned long long mh[kBins];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int c0 = c * kChunk;
  // The chunk's scores (up to the end of the row) and the maximum go out
  // together with the sequence's parameters; entries at or past L are ignored.
  const float* srow = a.scores + (size_t)u * a.score_ld;
  float v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int t = c0 + threadIdx.x + k * kNT;
    v[k] = t < a.score_ld ? srow[t] : 0.0f;
  }
  const uint32_t maxkey = a.maxkey[u];
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b);
  if (c0 >= p.L || p.dense || p.k_eff == 0) return;  // uniform over the workgroup
  const float M = key_to_float(maxkey);
  for (int i = threadIdx.x; i < kBins; i += kNT) mh[i] = 0ull;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int t = c0 + threadIdx.x + k * kNT;
    const unsigned long long q = mass_units(sexp(v[k] - M));
    if (t < p.L && q != 0ull) atomicAdd(&mh[order_key(v[k]) >> kDigit1Shift], q);
  }
  __syncthreads();
  unsigned long long* g = a.hist1m + (size_t)u * kBins;
  for (int i = threadIdx.x; i < kBins; i += kNT) {
    const unsigned long long q = mh[i];
    if (q != 0ull) atomicAdd(&g[i], q);
  }
}

// ------------------------------------------------------------------ threshold
// Per unit, from the first-digit histograms: the digit where the stratum
// ends (count rank k, or with top-p whichever of rank k and the mass target
// comes first) and a lower bound of W.  Every token whose first digit is
// below b1 is a tail token and its key is at least the smallest key of its
// digit, so
//   W >= sum_{digit < b1} count(digit) * exp(lowest score of digit - M);
// the sum uses the specified exp (monotone up to ~1 ulp) and is shrunk by
// 2^-10 to absorb that and the final rounding.
__global__ __launch_bounds__(kNT) void threshold_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ unsigned long long mh[kBins];
  __shared__ int scan_scr[kNT / 64];
  __shared__ int pair[2];
  __shared__ unsigned long long scan_m[kNT / 64];
  __shared__ unsigned long long pair_m[2];
  __shared__ double dscr[kNT / 64];
  const int u = blockIdx.x;
  // The histogram and the maximum depend on the unit only: their loads go
  // out together with the sequence's parameters.
  constexpr int kH = kBins / kNT;
  uint32_t hv[kH];
#pragma unroll
  for (int j = 0; j < kH; ++j) hv[j] = a.hist1[(size_t)u * kBins + threadIdx.x + j * kNT];
  const uint32_t maxkey = a.maxkey[u];
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b);
  if (p.dense || p.L == 0) {
    if (threadIdx.x == 0) a.thresh[u] = Thresh1{kBins, 0, 0.0f, 0, 0ull, 0, 0};
    return;
  }
  const bool topp = p.topp && p.k_eff > 0;
#pragma unroll
  for (int j = 0; j < kH; ++j) hist[threadIdx.x + j * kNT] = hv[j];
  if (topp)
    for (int i = threadIdx.x; i < kBins; i += kNT) mh[i] = a.hist1m[(size_t)u * kBins + i];
  __syncthreads();
  DigitBound d{kBins, 0, 0ull, 0};
  int bc = kBins, rc = 0;  // where the count bound ends (its rank search)
  if (p.k_eff > 0) {
    find_rank_bin<kNT>(hist, kBins, p.k_eff, scan_scr, pair, &bc, &rc);
    d = DigitBound{bc, rc, 0ull, kBoundCount};
    if (topp) {
      unsigned long long qs = 0ull;
      for (int i = threadIdx.x; i < kBins; i += kNT) qs += mh[i];
      const unsigned long long tau = mass_target(p.p, block_sum_u64<kNT>(qs, scan_m));
      if (tau == 0ull) {
        d = DigitBound{kBins, 0, 0ull, 0};
      } else {
        int bm;
        unsigned long long rm;
        find_bin<kNT>(mh, kBins, tau, scan_m, pair_m, &bm, &rm);
        d = combine_bounds(kBoundCount | kBoundMass, bc, rc, bm, rm);
      }
    }
  }
  const int b1 = d.bin;
  // Tokens above b1: the rank search already counted them when it chose b1.
  const int above = b1 == kBins ? 0
                    : (b1 == bc && (d.mode & kBoundCount)) ? p.k_eff - rc
                                                            : count_above<kNT>(hist, kBins, b1, scan_scr);
  const float M = key_to_float(maxkey);
  double lb = 0.0;
  for (int bin = threadIdx.x; bin < b1; bin += kNT) {
    const uint32_t n = hist[bin];
    const float lo = key_to_float((uint32_t)bin << kDigit1Shift);
    if (n && lo == lo) lb += (double)n * (double)sexp(lo - M);
  }
  lb = block_sum_f64<kNT>(lb, dscr);
  float wlb = (float)(lb * (1.0 - 0x1.0p-10));
  if (a.w_in) wlb = fminf(wlb, a.w_in[u]);
  if (threadIdx.x == 0) a.thresh[u] = Thresh1{b1, d.rem, wlb, d.mode, d.rem_mass, above, 0};
}

// ------------------------------------------------------------------ filter
// Per chunk: tokens whose first digit is above b1 are listed (deterministic
// set); tokens on b1 become candidates (index order, second-digit histogram);
// tokens below b1 are tail tokens: their weights are summed in fp64 for W and
// those passing the necessary inclusion test are listed with their weight.
// At most 64 VGPRs: eight waves per SIMD, so a 1M-token layer's chunk
// workgroups are all resident at once.
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(8))) void filter_kernel(
    SelectArgs a) {
  __shared__ float sh[kChunk];
  __shared__ int scan_scr[kNT / 64];
  __shared__ double dscr[kNT / 64];

  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int c0 = c * kChunk;
  // The chunk's scores, the threshold and the maximum depend on the unit and
  // chunk only: their loads go out together with the sequence's parameters.
  // Scores are read up to the end of the row (score_ld entries); entries at
  // or past L are ignored.  Each thread takes its 16 consecutive scores as
  // four 16-byte loads when the rows allow it (the fused path's always do);
  // otherwise they go through the LDS buffer with coalesced 4-byte loads
  // after the checks.
  const float* srow = a.scores + (size_t)u * a.score_ld;
  const bool direct = ((reinterpret_cast<uintptr_t>(srow) & 15u) | (a.score_ld & 3)) == 0;
  const int tb = threadIdx.x * kPer;
  float4 s4[kPer / 4];
  if (direct) {
#pragma unroll
    for (int g = 0; g < kPer / 4; ++g) {
      // Unconditional loads (clamped into the row) keep the four in flight
      // together; a row holds at least 4 entries here.
      const int t = c0 + tb + 4 * g;
      s4[g] = *reinterpret_cast<const float4*>(srow + (t < a.score_ld ? t : 0));
    }
  }
  const Thresh1 t1 = a.thresh[u];
  const uint32_t maxkey = a.maxkey[u];
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const int h = ui.h;
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b);
  if (c0 >= p.L || p.dense) return;  // uniform over the workgroup
  const float M = key_to_float(maxkey);
  if (!direct) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int t = c0 + threadIdx.x + k * kNT;
      sh[threadIdx.x + k * kNT] = srow[t < a.score_ld ? t : a.score_ld - 1];
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kPer / 4; ++g) s4[g] = *reinterpret_cast<const float4*>(sh + tb + 4 * g);
  }
  filter_chunk(a, p, t1, M, u, b, h, ui.grp, c, s4, sh, scan_scr, dscr);
}

// ------------------------------------------------------------------ resolve
// One workgroup per unit: finish the radix select on the candidates (second
// digit from the histogram, third digit from an LDS histogram of the
// candidates sharing the first two digits), then the per-chunk tie counts,
// the tie quota offsets and the tail normaliser W.  Candidate passes run over
// the flattened candidate list, every thread on a fixed stride, so loads are
// independent and every sum has a fixed order.
constexpr int kRT = 1024;
constexpr int kRW = kRT / 64;
constexpr int kMaxResolveChunks = SSA_MAX_SEQ_LEN / kChunk;
static_assert(kBins % kRT == 0, "each resolve thread loads kBins / kRT histogram entries");

// Candidate passes: thread t serves chunk (t / tpc) + k * (kRT / tpc) and,
// inside it, items (t % tpc) + i * tpc.  Every load is independent and every
// thread's items are fixed by (nc, t): sums over them have a fixed order.
__device__ __forceinline__ int threads_per_chunk(int nc) {
  int tpc = kRT;
  while (tpc > 1 && tpc * nc > kRT) tpc >>= 1;
  return tpc;
}

// Early stopping: where each chunk's words above the threshold key (its
// listed tokens above the threshold digit, then its candidates above the key;
// packed << 16 in cnt) start in the unit's word array, and their total.
__device__ __forceinline__ void stop_offsets(const SelectArgs& a, int u, size_t cu, int nc,
                                          const int* cnt, int* scan_scr) {
  int run = 0;
  for (int c0 = 0; c0 < nc; c0 += kRT) {
    const int c = c0 + threadIdx.x;
    const int w = c < nc ? clamp_count(a.list_cnt[2 * (cu + c)], kChunk) + (cnt[c] >> 16) : 0;
    int tot;
    const int ex = block_exclusive_scan<kRT>(w, scan_scr, &tot);
    if (c < nc) a.stop_off[cu + c] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) a.stop_n[u] = run;
}

__global__ __launch_bounds__(kRT) void resolve_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ unsigned long long mh[kBins];  // mass units per digit (top-p)
  __shared__ int ties_sh[kMaxResolveChunks];  // ties + (candidates above the key << 16)
  __shared__ int scan_scr[kRW];
  __shared__ int pair[2];
  __shared__ unsigned long long scan_m[kRW];
  __shared__ unsigned long long pair_m[2];
  __shared__ double dscr[kRW];

  const int u = blockIdx.x;
  // Every load that depends on the unit only is issued first, together: the
  // sequence's parameters, the first-digit threshold and the maximum, the
  // second-digit histogram, and this thread's candidate count and first
  // candidate keys (read whole within the chunk's segment; entries past the
  // count are never used).  Candidate passes give tpc threads to each chunk,
  // fixed by the launch's chunk count, so every thread's items and every sum
  // have a fixed order.
  constexpr int kKeep = 16;
  constexpr int kHist = kBins / kRT;
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b);
  const Thresh1 t1 = a.thresh[u];
  const uint32_t maxkey = a.maxkey[u];
  uint32_t hv[kHist];
#pragma unroll
  for (int j = 0; j < kHist; ++j) hv[j] = a.hist2[(size_t)u * kBins + threadIdx.x + j * kRT];
  const size_t cu = (size_t)u * a.nchunk;
  const uint32_t* ckeys = a.cand_key + (size_t)u * a.seg_ld;
  const int tpc = threads_per_chunk(a.nchunk);
  const int cstep = kRT / tpc;
  const int csub = threadIdx.x % tpc;
  const bool one_chunk = a.nchunk <= cstep;  // each thread serves at most one chunk
  const int cm = threadIdx.x / tpc;
  const bool has_cm = one_chunk && cm < a.nchunk;
  const int cnt_m = has_cm ? a.cand_cnt[cu + cm] : 0;
  const uint32_t* ckm = ckeys + (size_t)cm * kChunk;
  uint32_t kr[kKeep];
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const int i = csub + k * tpc;
    kr[k] = (has_cm && i < kChunk) ? ckm[i] : 0u;
  }
  UnitState st;
  st.tkey = 0u;
  st.ties_needed = 0;
  st.M = 0.0f;
  st.W = 0.0f;
  st.flags = 0;
  st.k_eff = p.k_eff;
  st.m = p.m;
  st.L = p.L;
  double W = 0.0;

  if (p.L == 0) {
    st.flags = kFlagEmpty;
  } else {
    st.M = key_to_float(maxkey);
    if (p.dense) {
      st.flags = kFlagDense;
    } else {
      const int nc = (p.L + kChunk - 1) / kChunk;
      // The chunks' tail sums do not depend on anything below: load them first.
      double acc = 0.0;
      for (int c = threadIdx.x; c < nc; c += kRT) acc += a.wpart[cu + c];
      double cs = 0.0;  // this thread's candidates below the threshold key
      int total_ties = 0;
      if (t1.mode == 0) {
        st.flags = kFlagNoTopk;
        st.k_eff = 0;
      } else {
        const int nm = (has_cm && cm < nc) ? clamp_count(cnt_m, kChunk) : 0;
#pragma unroll
        for (int j = 0; j < kHist; ++j) hist[threadIdx.x + j * kRT] = hv[j];
        if (t1.mode & kBoundMass)
          for (int i = threadIdx.x; i < kBins; i += kRT) mh[i] = a.hist2m[(size_t)u * kBins + i];
        for (int c = threadIdx.x; c < nc; c += kRT) ties_sh[c] = 0;
        __syncthreads();
        // Second digit.
        // The candidates above the chosen bin: counted by the rank search when
        // the count bound chose it.
        DigitBound d2;
        int above2;
        {
          int bc = 0, rc = 0, bm = 0;
          unsigned long long rm = 0ull;
          if (t1.mode & kBoundCount) find_rank_bin<kRT>(hist, kBins, t1.rem, scan_scr, pair, &bc, &rc);
          if (t1.mode & kBoundMass) find_bin<kRT>(mh, kBins, t1.rem_mass, scan_m, pair_m, &bm, &rm);
          d2 = combine_bounds(t1.mode, bc, rc, bm, rm);
          above2 = ((d2.mode & kBoundCount) && d2.bin == bc)
                       ? t1.rem - rc
                       : count_above<kRT>(hist, kBins, d2.bin, scan_scr);
        }
        const bool mass3 = d2.mode & kBoundMass;
        const uint32_t prefix = ((uint32_t)t1.b1 << 11) | (uint32_t)d2.bin;
        for (int i = threadIdx.x; i < kBins3; i += kRT) {
          hist[i] = 0u;
          if (mass3) mh[i] = 0ull;
        }
        __syncthreads();
        // Third digit: LDS histograms of the candidates that share the prefix.
        auto add3 = [&](uint32_t key) {
          if ((key >> kDigit2Shift) == prefix) {
            atomicAdd(&hist[key & (kBins3 - 1)], 1u);
            if (mass3) atomicAdd(&mh[key & (kBins3 - 1)], mass_units(sexp(key_to_float(key) - st.M)));
          }
        };
        if (one_chunk) {
#pragma unroll
          for (int k = 0; k < kKeep; ++k) {
            const int i = csub + k * tpc;
            if (i < nm) add3(kr[k]);
          }
          for (int i = csub + kKeep * tpc; i < nm; i += tpc) add3(ckm[i]);
        } else {
          for (int c = threadIdx.x / tpc; c < nc; c += cstep) {
            const int n = clamp_count(a.cand_cnt[cu + c], kChunk);
            const uint32_t* ck = ckeys + (size_t)c * kChunk;
            for (int i = csub; i < n; i += tpc) add3(ck[i]);
          }
        }
        __syncthreads();
        DigitBound d3;
        int above3;
        {
          int bc = 0, rc = 0, bm = 0;
          unsigned long long rm = 0ull;
          if (d2.mode & kBoundCount) find_rank_bin<kRT>(hist, kBins3, d2.rem, scan_scr, pair, &bc, &rc);
          if (mass3) find_bin<kRT>(mh, kBins3, d2.rem_mass, scan_m, pair_m, &bm, &rm);
          d3 = combine_bounds(d2.mode, bc, rc, bm, rm);
          above3 = ((d3.mode & kBoundCount) && d3.bin == bc)
                       ? d2.rem - rc
                       : count_above<kRT>(hist, kBins3, d3.bin, scan_scr);
        }
        st.tkey = (prefix << kDigit2Shift) | (uint32_t)d3.bin;
        // Tokens on the last key all carry the same mass: the mass bound needs
        // ceil(remaining units / units per token) of them.
        int need = d3.rem;
        if (d3.mode & kBoundMass) {
          const unsigned long long qT = mass_units(sexp(key_to_float(st.tkey) - st.M));
          const unsigned long long nmass = qT ? (d3.rem_mass + qT - 1ull) / qT : 1ull;
          need = (d3.mode & kBoundCount) ? (int)min((unsigned long long)need, nmass) : (int)nmass;
        }
        st.ties_needed = need;
        st.k_eff = t1.above + above2 + above3 + need;
        // Ties on the threshold key per chunk and candidates above it
        // (integer, packed as ties + (above << 16): each at most 4096), and
        // the weight of the candidates strictly below it (each thread over
        // its fixed items, in order; summed with the chunk sums below).
        if (one_chunk) {
          int ties = 0;
#pragma unroll
          for (int k = 0; k < kKeep; ++k) {
            const int i = csub + k * tpc;
            if (i < nm) {
              ties += kr[k] == st.tkey ? 1 : (kr[k] > st.tkey ? 0x10000 : 0);
              if (kr[k] < st.tkey) cs += (double)sexp(key_to_float(kr[k]) - st.M);
            }
          }
          for (int i = csub + kKeep * tpc; i < nm; i += tpc) {
            const uint32_t key = ckm[i];
            ties += key == st.tkey ? 1 : (key > st.tkey ? 0x10000 : 0);
            if (key < st.tkey) cs += (double)sexp(key_to_float(key) - st.M);
          }
          if (ties) atomicAdd(&ties_sh[cm], ties);
        } else {
          for (int c = threadIdx.x / tpc; c < nc; c += cstep) {
            const int n = clamp_count(a.cand_cnt[cu + c], kChunk);
            const uint32_t* ck = ckeys + (size_t)c * kChunk;
            int ties = 0;
            for (int i = csub; i < n; i += tpc) {
              const uint32_t key = ck[i];
              ties += key == st.tkey ? 1 : (key > st.tkey ? 0x10000 : 0);
              if (key < st.tkey) cs += (double)sexp(key_to_float(key) - st.M);
            }
            if (ties) atomicAdd(&ties_sh[c], ties);
          }
        }
        __syncthreads();  // the chunks' tie counts are complete
        int run = 0;
        for (int c0 = 0; c0 < nc; c0 += kRT) {
          const int c = c0 + threadIdx.x;
          const int v = c < nc ? ties_sh[c] & 0xffff : 0;
          int tot;
          const int ex = block_exclusive_scan<kRT>(v, scan_scr, &tot);
          if (c < nc) {
            a.ties_before[cu + c] = run + ex;
            a.tiecnt[cu + c] = v;
          }
          run += tot;
        }
        total_ties = run;
        if (a.stop_off) stop_offsets(a, u, cu, nc, ties_sh, scan_scr);
      }
      W = block_sum_f64<kRT>(acc + cs, dscr);  // every thread's share, one fixed tree
      if (t1.mode != 0) {
        const double wT = (double)sexp(key_to_float(st.tkey) - st.M);
        W += (double)(total_ties - st.ties_needed) * wT;
      }
      // With a top-p mass the dense rule (k + m >= L) is only decidable now.
      if (p.topp && (int64_t)st.k_eff + (int64_t)p.m >= (int64_t)p.L) {
        st.flags = kFlagDense;
        W = 0.0;
      }
    }
  }
  st.W = a.w_in ? a.w_in[u] : (float)W;
  if (!(st.flags & (kFlagEmpty | kFlagDense)) && p.m > 0 && p.L - st.k_eff > 0 && st.W > 0.0f)
    st.flags |= kFlagSample;
  if (threadIdx.x == 0) {
    reinterpret_cast<UnitState*>(a.state)[u] = st;
    if (a.norm_out) {
      a.norm_out[2 * u] = st.M;
      a.norm_out[2 * u + 1] = st.W;
    }
  }
}

// ------------------------------------------------------------------ early stopping
// "S2O: Early Stopping for Sparse Attention via Online Permutation",
// methodology part 2.  The deterministic stratum, in its order (key
// descending, position ascending), is cut into 64-token blocks whose gains are
// their mass units; the visit stops after the first block whose gain is below
// tau times the mass so far (exact integer arithmetic).  A token's word is
// ((~key) << 32) | position, so ascending words are the stratum's order, and
// the cut is published as the last word kept: the sample kernel drops every
// deterministic token whose word is larger.  The stratum is the tokens above
// the threshold key T (at most 16384 when a cut applies) followed by the
// first ties on T (one mass value, ranked by position), so only the former
// are ordered, in five steps that spread over the device and use no global
// atomics:
//   stop_gather: each chunk writes its words above T (its listed tokens
//     above the threshold digit, then its candidates above T) at the offset
//     the resolve kernel computed for it;
//   stop_sort: one workgroup sorts each 1024-word slice (4 words per thread
//     in registers, cross-wave exchanges through LDS);
//   stop_pair: for every pair of slices, the number of words of one below
//     each word of the other (searched in LDS), one count array per pair;
//   stop_final: each word's rank = its index in its slice + those counts;
//     mass and word stored in rank order;
//   stop_cut: one workgroup per unit sums the block gains (ties count at
//     T's mass), scans them, finds the stop and writes the last word kept.
constexpr int kStopBlock = 64;
constexpr int kStopMax = 16384;  // largest stratum that is truncated
constexpr int kSlice = 1024;     // words sorted per wave
constexpr int kSlices = kStopMax / kSlice;
constexpr int kSortT = 256;                // threads per slice sort
constexpr int kSE = kSlice / kSortT;      // words per thread in the sort

// gain < tau * acc, exactly, for 0 < tau (tau >= 1 compares with acc).
__device__ __forceinline__ bool gain_below(unsigned long long gain, unsigned long long acc,
                                           float tau) {
  if (tau >= 1.0f) return gain < acc;
  int e;
  const float f = __builtin_frexpf(tau, &e);
  const unsigned long long mant = (unsigned long long)(f * 0x1.0p24f);  // tau = mant 2^(e-24)
  const unsigned __int128 rhs = (unsigned __int128)mant * acc;          // < 2^86
  const int D = 24 - e;                                                 // >= 24
  if (gain == 0ull) return rhs != 0;
  if (D >= 86 || (64 - __builtin_clzll(gain)) + D > 127) return false;  // lhs >= 2^86 > rhs
  return ((unsigned __int128)gain << D) < rhs;
}

// Whether early stopping can cut this unit's stratum (uniform per unit).
__device__ __forceinline__ bool stop_applies(const UnitState& st) {
  if (st.flags & (kFlagEmpty | kFlagDense | kFlagNoTopk)) return false;
  return st.k_eff > kStopBlock && st.k_eff <= kStopMax;
}

__device__ __forceinline__ unsigned long long stratum_word(uint32_t key, int pos) {
  return ((unsigned long long)~key << 32) | (uint32_t)pos;
}

// The value of lane ^ L, for a compile-time L < 64: lane distances 1 and 2
// are quad permutations and 8 a rotation by 8 within a row of 16 (DPP, plain
// VALU moves); 4 and 16 are swizzles within 32 lanes; 32 goes through the LDS
// crossbar.
template <int L>
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16 || L == 32, "lane distance");
  if constexpr (L == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  } else if constexpr (L == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  } else if constexpr (L == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);  // row_ror 8
  } else if constexpr (L == 4 || L == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (L << 10));  // xor within 32
  } else {
    return (uint32_t)__shfl_xor((int)x, L);
  }
}

template <int L>
__device__ __forceinline__ unsigned long long lane_xor64(unsigned long long x) {
  const uint32_t lo = lane_xor32<L>((uint32_t)x);
  const uint32_t hi = lane_xor32<L>((uint32_t)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// One bitonic stage (merge size K, partner distance J) on N = NT * E words
// held E per thread in registers (element i = E * tid + e).  K and J are
// compile-time constants, so every branch below folds: pairs closer than E
// are exchanged inside a thread, pairs closer than 64 E across the lanes of a
// wave by shuffle, the rest through LDS (buf: element E t + e at e * NT + t,
// consecutive words per wave: no bank conflicts).
template <int NT, int E, int K, int J>
__device__ __forceinline__ void bitonic_stage(unsigned long long (&v)[E], unsigned long long* buf,
                                              int tid) {
  if constexpr (J < E) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & J) != 0) continue;
      // ascending iff bit K of the element index is clear
      const bool asc = K >= E ? ((E * tid) & K) == 0 : (e & K) == 0;
      const unsigned long long x = v[e], y = v[e + J];
      const bool swap = asc == (x > y);
      v[e] = swap ? y : x;
      v[e + J] = swap ? x : y;
    }
  } else {
    // J >= E: the partner is element i ^ J, in thread tid ^ (J / E), same
    // register; this thread keeps the minimum iff bit J and bit K of its
    // element indices agree (both depend on tid only).
    const bool keep_min = (((E * tid) & J) == 0) == (((E * tid) & K) == 0);
    if constexpr (J >= E * 64) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) buf[e * NT + tid] = v[e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned long long o = buf[e * NT + (tid ^ (J / E))];
        v[e] = keep_min == (o < v[e]) ? o : v[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned long long o = lane_xor64<J / E>(v[e]);
        v[e] = keep_min == (o < v[e]) ? o : v[e];
      }
    }
  }
}

template <int NT, int E, int K, int J>
__device__ __forceinline__ void bitonic_merge(unsigned long long (&v)[E], unsigned long long* buf,
                                              int tid) {
  bitonic_stage<NT, E, K, J>(v, buf, tid);
  if constexpr (J > 1) bitonic_merge<NT, E, K, J / 2>(v, buf, tid);
}

// Bitonic sort, ascending, of NT * E words (element i = E * tid + e).
template <int NT, int E, int K = 2>
__device__ __forceinline__ void bitonic_sort(unsigned long long (&v)[E], unsigned long long* buf,
                                             int tid) {
  bitonic_merge<NT, E, K, K / 2>(v, buf, tid);
  if constexpr (K < NT * E) bitonic_sort<NT, E, K * 2>(v, buf, tid);
}

// Grid: (chunks, units) x kNT threads.
__global__ __launch_bounds__(kNT) void stop_gather_kernel(SelectArgs a) {
  __shared__ int scan_scr[kNT / 64];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  if (!stop_applies(st)) return;  // uniform
  const int c0 = c * kChunk;
  if (c0 >= st.L) return;  // uniform
  const int n_words = min(max(a.stop_n[u], 0), kStopMax);
  const size_t ci = (size_t)u * a.nchunk + c;
  const size_t seg = (size_t)u * a.seg_ld + c0;
  const int off = a.stop_off[ci];
  const int n_above = clamp_count(a.list_cnt[2 * ci], kChunk);
  const int ncand = clamp_count(a.cand_cnt[ci], kChunk);
  const int nvalid = min(kChunk, st.L - c0);
  const float* srow = a.scores + (size_t)u * a.score_ld;
  unsigned long long* out = a.stop_words + (size_t)u * kStopMax;
  for (int i = threadIdx.x; i < n_above; i += kNT) {
    const int pos = c0 + min(max(a.list_idx[seg + i] - c0, 0), nvalid - 1);
    const int at = off + i;
    if (at >= 0 && at < n_words) out[at] = stratum_word(order_key(srow[pos]), pos);
  }
  // Candidates above T, compacted in list (position) order.
  int run = off + n_above;
  for (int base = 0; base < ncand; base += kNT) {
    const int i = base + threadIdx.x;
    const uint32_t key = i < ncand ? a.cand_key[seg + i] : 0u;
    const bool in = i < ncand && key > st.tkey;
    int tot;
    const int at = run + block_exclusive_scan<kNT>(in ? 1 : 0, scan_scr, &tot);
    if (in && at >= 0 && at < n_words) {
      const int pos = c0 + min(max(a.cand_idx[seg + i] - c0, 0), nvalid - 1);
      out[at] = stratum_word(key, pos);
    }
    run += tot;
  }
}

// Grid: (kSlices, units) x kSortT threads.
__global__ __launch_bounds__(kSortT) void stop_sort_kernel(SelectArgs a) {
  __shared__ unsigned long long buf[kSlice];
  const int u = blockIdx.y;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  if (!stop_applies(st)) return;  // uniform
  const int n_words = min(max(a.stop_n[u], 0), kStopMax);
  const int f0 = blockIdx.x * kSlice;
  if (f0 >= n_words) return;  // uniform
  const int tid = threadIdx.x;
  unsigned long long* w = a.stop_words + (size_t)u * kStopMax + f0;
  unsigned long long v[kSE];
#pragma unroll
  for (int e = 0; e < kSE; ++e) {  // the start order is free: coalesced loads
    const int f = e * kSortT + tid;
    v[e] = f0 + f < n_words ? w[f] : ~0ull;  // padding sorts last
  }
  bitonic_sort<kSortT, kSE>(v, buf, tid);
#pragma unroll
  for (int e = 0; e < kSE; ++e) w[kSE * tid + e] = v[e];
}

// Grid: (kSlices * kSlices, units) x kNT threads: block (s, o) counts, for
// each word of slice o, the words of slice s below it.
__global__ __launch_bounds__(kNT) void stop_pair_kernel(SelectArgs a) {
  constexpr int E = kSlice / kNT;
  __shared__ unsigned long long sw[kSlice];
  const int u = blockIdx.y;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  if (!stop_applies(st)) return;  // uniform
  const int n_words = min(max(a.stop_n[u], 0), kStopMax);
  const int ns = (n_words + kSlice - 1) / kSlice;
  const int s = blockIdx.x % kSlices;
  const int o = blockIdx.x / kSlices;
  if (s >= ns || o >= ns || s == o) return;  // uniform
  const unsigned long long* words = a.stop_words + (size_t)u * kStopMax;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < E; ++e) sw[e * kNT + tid] = words[s * kSlice + e * kNT + tid];
  unsigned long long x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = words[o * kSlice + E * tid + e];
  __syncthreads();
  // branchless binary searches, the thread's E searches stepping together
  int lb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) lb[e] = 0;
#pragma unroll
  for (int step = kSlice / 2; step >= 1; step >>= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) lb[e] += sw[lb[e] + step - 1] < x[e] ? step : 0;
  }
  uint16_t* cnt = a.stop_pair + (((size_t)u * kSlices + o) * kSlices + s) * kSlice + E * tid;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt[e] = (uint16_t)(lb[e] + (sw[lb[e]] < x[e] ? 1 : 0));
}

// Grid: (kSlices, units) x kNT threads.
__global__ __launch_bounds__(kNT) void stop_final_kernel(SelectArgs a) {
  constexpr int E = kSlice / kNT;
  static_assert(E == 4, "four 16-bit counts per 8-byte load");
  const int u = blockIdx.y;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  if (!stop_applies(st)) return;  // uniform
  const int n_words = min(max(a.stop_n[u], 0), kStopMax);
  const int ns = (n_words + kSlice - 1) / kSlice;
  const int o = blockIdx.x;
  if (o >= ns) return;  // uniform
  const int tid = threadIdx.x;
  const unsigned long long* words = a.stop_words + (size_t)u * kStopMax + o * kSlice;
  unsigned long long x[E];
  int rank[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = words[E * tid + e];
    rank[e] = E * tid + e;  // words of its own slice below it
  }
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {  // fixed trip count: all count loads in flight
    if (s < ns && s != o) {
      const uint16_t* cnt =
          a.stop_pair + (((size_t)u * kSlices + o) * kSlices + s) * kSlice + E * tid;
      const uint2 c4 = *reinterpret_cast<const uint2*>(cnt);  // E = 4 counts
      rank[0] += c4.x & 0xffffu;
      rank[1] += c4.x >> 16;
      rank[2] += c4.y & 0xffffu;
      rank[3] += c4.y >> 16;
    }
  }
  unsigned long long* mass = a.stop_mass + (size_t)u * kStopMax;
  unsigned long long* rword = a.stop_rword + (size_t)u * kStopMax;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // words are distinct, so ranks are: a permutation of [0, n_words)
    if (x[e] != ~0ull && rank[e] < n_words) {
      const uint32_t key = ~(uint32_t)(x[e] >> 32);
      mass[rank[e]] = mass_units(sexp(key_to_float(key) - st.M));
      rword[rank[e]] = x[e];
    }
  }
}

// Grid: units x kNT threads (one per 64-token block of the largest stratum).
__global__ __launch_bounds__(kNT) void stop_cut_kernel(SelectArgs a) {
  constexpr int kNB = kStopMax / kStopBlock;
  static_assert(kNB == kNT, "one thread per block of the largest stratum");
  __shared__ unsigned long long scan_m[kNT / 64];
  __shared__ int scan_scr[kNT / 64];
  __shared__ int first_sh;
  __shared__ int tie_pos_sh;
  const int u = blockIdx.x;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  const int tid = threadIdx.x;
  if (!stop_applies(st)) {  // uniform
    if (tid == 0) a.stop_cut[u] = ~0ull;
    return;
  }
  const int n = st.k_eff;
  const int n_words = min(min(max(a.stop_n[u], 0), kStopMax), n);  // ranks below: words above T
  const unsigned long long qT = mass_units(sexp(key_to_float(st.tkey) - st.M));
  const int nb = (n + kStopBlock - 1) / kStopBlock;
  if (tid == 0) {
    first_sh = 0x7fffffff;
    tie_pos_sh = 0;
  }
  unsigned long long g = 0ull;
  if (tid < nb) {
    // The block's masses: 32 16-byte loads, all in flight together.
    const unsigned long long* mass = a.stop_mass + (size_t)u * kStopMax;
    const int r0 = tid * kStopBlock;
    const int r1 = min(r0 + kStopBlock, n);
#pragma unroll
    for (int q = 0; q < kStopBlock / 2; ++q) {
      const int r = r0 + 2 * q;
      if (r < n_words) {
        const ulonglong2 m2 = *reinterpret_cast<const ulonglong2*>(mass + r);
        g += m2.x + (r + 1 < n_words ? m2.y : 0ull);
      }
    }
    if (r1 > n_words) g += (unsigned long long)(r1 - max(r0, n_words)) * qT;  // ties on T
  }
  unsigned long long tot;
  const unsigned long long acc = block_exclusive_scan<kNT>(g, scan_m, &tot) + g;
  if (tid < nb && gain_below(g, acc, a.stop_tau)) atomicMin(&first_sh, tid);
  __syncthreads();
  const int kept = first_sh == 0x7fffffff ? n : min(n, (first_sh + 1) * kStopBlock);
  unsigned long long cut = ~0ull;  // nothing cut
  if (kept < n) {
    if (kept <= n_words) {
      cut = a.stop_rword[(size_t)u * kStopMax + kept - 1];
    } else {
      // The cut falls among the ties on T: tie number t (in position order)
      // is the last one kept.  Find its chunk, then its place in the chunk's
      // candidate list (position order).
      const int t = kept - n_words - 1;
      const size_t cu = (size_t)u * a.nchunk;
      const int nc = (st.L + kChunk - 1) / kChunk;
      for (int c = 0; c < nc; ++c) {  // uniform loop; each chunk's test is uniform
        const int tb = a.ties_before[cu + c];
        const int tc = a.tiecnt[cu + c];
        if (t < tb || t >= tb + tc) continue;
        const int ncand = clamp_count(a.cand_cnt[cu + c], kChunk);
        const size_t seg = (size_t)u * a.seg_ld + (size_t)c * kChunk;
        int run = tb;
        for (int base = 0; base < ncand; base += kNT) {
          const int i = base + tid;
          const bool tie = i < ncand && a.cand_key[seg + i] == st.tkey;
          int ntie;
          const int r = run + block_exclusive_scan<kNT>(tie ? 1 : 0, scan_scr, &ntie);
          if (tie && r == t) tie_pos_sh = min(max(a.cand_idx[seg + i], 0), st.L - 1);
          run += ntie;
        }
        break;
      }
      __syncthreads();
      cut = stratum_word(st.tkey, tie_pos_sh);
    }
  }
  if (tid == 0) a.stop_cut[u] = cut;
}

// ------------------------------------------------------------------ sample
// Per chunk: membership of the listed tokens only -- above-threshold tokens
// and candidates above the threshold key (or within the tie quota) form the
// deterministic set; the other candidates and the listed sampling candidates
// take the exact inclusion test with the final W.  The chunk's segment is then
// written from an LDS membership map: deterministic tokens ascending, then
// sampled tokens ascending.  With emit_rows the segment holds cache row
// numbers (for the fused attention stage) instead of positions.
// Membership of a chunk position: not selected, deterministic, or sampled
// with its logit bias -log(pi) stored as the word itself (a finite float,
// never one of the two marks, which are NaN patterns).
constexpr uint32_t kMarkNone = 0xffffffffu;
constexpr uint32_t kMarkDet = 0xfffffffeu;

__device__ __forceinline__ void sample_one(const UnitState& st, uint64_t seed, int b, int h,
                                           int grp, int t, float w, int c0, int nvalid,
                                           uint32_t* mark) {
  if ((unsigned)(t - c0) >= (unsigned)nvalid) return;  // not a position of this chunk
  const uint4 wd = philox_block(seed, b, h, (uint32_t)t >> 2, grp);
  const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
  const float mw = (float)st.m * w;
  if (uniform24(words[t & 3]) * st.W < mw)
    mark[t - c0] = __float_as_uint(-logf(fminf(1.0f, mw / st.W)));
}

__global__ __launch_bounds__(kNT) void sample_kernel(SelectArgs a) {
  __shared__ uint32_t mark[kChunk];  // kMarkNone, kMarkDet or a sampled token's bias
  __shared__ int scan_scr[kNT / 64];
  static_assert(kPer == kBlockTokens, "a thread's positions are one cache block");

  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const int h = ui.h;
  const int c0 = c * kChunk;
  const size_t ci = (size_t)u * a.nchunk + c;
  const int tid = threadIdx.x;
  // Independent loads first: unit state, per-chunk counts, the chunk's block
  // ids, and this thread's first entry of each list (the lists are read
  // whole within the chunk's segment; entries past a count are never used),
  // so the common chunk, with fewer than kNT entries per list, needs no
  // further round trip.
  const int32_t* lidx = a.list_idx + (size_t)u * a.seg_ld + c0;
  const float* lw = a.list_w + (size_t)u * a.seg_ld + c0;
  const int32_t* cidx = a.cand_idx + (size_t)u * a.seg_ld + c0;
  const uint32_t* ckey = a.cand_key + (size_t)u * a.seg_ld + c0;
  const int l_first = lidx[tid];
  const float w_first = lw[tid];
  const int c_first = cidx[tid];
  const uint32_t k_first = ckey[tid];
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  // Counts are clamped to the segment and positions checked against the
  // chunk, so no value in the workspace can address outside it.
  const int n_above = clamp_count(a.list_cnt[2 * ci], kChunk);
  const int n_samp = clamp_count(a.list_cnt[2 * ci + 1], kChunk - n_above);
  const int ncand = clamp_count(a.cand_cnt[ci], kChunk);
  const int before = a.ties_before[ci];
  const uint64_t seed = a.seed[b];
  int32_t* cnt = a.sel_cnt + ci * 2;
  if (c0 >= st.L || (st.flags & kFlagEmpty)) {
    if (threadIdx.x == 0) {
      cnt[0] = 0;
      cnt[1] = 0;
    }
    return;
  }
  const int nvalid = min(kChunk, st.L - c0);
  const bool dense = st.flags & kFlagDense;
  const bool sampling = st.flags & kFlagSample;
  // This thread's positions are one cache block: its id, for emitted rows.
  int blk = 0;
  if (a.emit_rows && threadIdx.x < (nvalid + kBlockTokens - 1) / kBlockTokens) {
    blk = a.block_table[(size_t)b * a.max_blocks + c0 / kBlockTokens + threadIdx.x];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
  }
  for (int i = threadIdx.x; i < kChunk; i += kNT)
    mark[i] = (dense && i < nvalid) ? kMarkDet : kMarkNone;
  // Early stopping: the last stratum word kept (~0: the whole stratum).
  const unsigned long long cut = a.stop_cut && !dense ? a.stop_cut[u] : ~0ull;
  __syncthreads();
  if (!dense) {
    const float* srow = a.scores + (size_t)u * a.score_ld;
    // The chunk's list: tokens above the threshold digit, then the listed
    // sampling candidates with their weights.
    const int n_list = n_above + (sampling ? n_samp : 0);
    for (int i = tid; i < n_list; i += kNT) {
      const int t = i == tid ? l_first : lidx[i];
      if (i < n_above) {
        if ((unsigned)(t - c0) < (unsigned)nvalid &&
            (cut == ~0ull || stratum_word(order_key(srow[t]), t) <= cut))
          mark[t - c0] = kMarkDet;
      } else {
        sample_one(st, seed, b, h, ui.grp, t, i == tid ? w_first : lw[i], c0, nvalid, mark);
      }
    }
    if (!(st.flags & kFlagNoTopk)) {
      // Threshold-digit candidates, in index order: key above T -> S; key == T
      // -> S while the tie quota lasts; otherwise a tail token.
      int run = 0;  // ties seen in earlier rounds of this loop
      for (int base = 0; base < ncand; base += kNT) {
        const int i = base + tid;
        const bool v = i < ncand;
        const uint32_t key = v ? (base == 0 ? k_first : ckey[i]) : 0u;
        const int t = v ? (base == 0 ? c_first : cidx[i]) : 0;
        const bool tie = v && key == st.tkey;
        int tot;
        const int rank = before + run + block_exclusive_scan<kNT>(tie ? 1 : 0, scan_scr, &tot);
        run += tot;
        if (v) {
          if (key > st.tkey || (tie && rank < st.ties_needed)) {
            // stratum tokens past the early stop are neither read nor sampled
            if ((unsigned)(t - c0) < (unsigned)nvalid && stratum_word(key, t) <= cut)
              mark[t - c0] = kMarkDet;
          } else if (sampling) {
            sample_one(st, seed, b, h, ui.grp, t, sexp(key_to_float(key) - st.M), c0, nvalid,
                       mark);
          }
        }
      }
    }
  }
  __syncthreads();
  // Compaction from the membership map (16 consecutive positions per thread).
  const int tb = threadIdx.x * kPer;
  uint32_t smask = 0u, rmask = 0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t m = mark[tb + i];
    smask |= (uint32_t)(m == kMarkDet) << i;
    rmask |= (uint32_t)(m < kMarkDet) << i;
  }
  // One scan for both counts: deterministic count in the low 16 bits,
  // sampled count in the high 16 bits (each at most 4096).
  int packed_tot;
  const int packed = block_exclusive_scan<kNT>(__popc(smask) | (__popc(rmask) << 16), scan_scr,
                                               &packed_tot);
  const int totS = packed_tot & 0xffff;
  const int totR = packed_tot >> 16;
  int32_t* sidx = a.sel_idx + (size_t)u * a.seg_ld + c0;
  float* slw = a.sel_logw + (size_t)u * a.seg_ld + c0;
  int ws = packed & 0xffff, wr = totS + (packed >> 16);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t bit = 1u << i;
    if ((smask | rmask) & bit) {
      const int t = c0 + tb + i;
      const int v = a.emit_rows ? (blk * a.Hkv + h) * kBlockTokens + (t & 15) : t;
      if (smask & bit) {
        sidx[ws] = v;
        slw[ws] = 0.0f;
        ++ws;
      } else {
        sidx[wr] = v;
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

// ------------------------------------------------------------------ test hooks

__global__ void debug_philox_kernel(uint64_t seed, int b, int h, int grp, int j0, int n,
                                    uint32_t* words) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t j = (uint32_t)(j0 + i);
  const uint4 wd = philox_block(seed, b, h, j >> 2, grp);
  const uint32_t w4[4] = {wd.x, wd.y, wd.z, wd.w};
  words[i] = w4[j & 3u];
}

__global__ void debug_sexp_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = sexp(x[i]);
}

}  // namespace

hipError_t launch_mass(const SelectArgs& a, int units, hipStream_t stream) {
  mass_kernel<<<dim3(a.nchunk, units), kNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_threshold(const SelectArgs& a, int units, hipStream_t stream) {
  threshold_kernel<<<units, kNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_filter(const SelectArgs& a, int units, hipStream_t stream) {
  filter_kernel<<<dim3(a.nchunk, units), kNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_resolve(const SelectArgs& a, int units, hipStream_t stream) {
  resolve_kernel<<<units, kRT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_stop(const SelectArgs& a, int units, hipStream_t stream) {
  stop_gather_kernel<<<dim3(a.nchunk, units), kNT, 0, stream>>>(a);
  stop_sort_kernel<<<dim3(kSlices, units), kSortT, 0, stream>>>(a);
  stop_pair_kernel<<<dim3(kSlices * kSlices, units), kNT, 0, stream>>>(a);
  stop_final_kernel<<<dim3(kSlices, units), kNT, 0, stream>>>(a);
  stop_cut_kernel<<<units, kNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_sample(const SelectArgs& a, int units, hipStream_t stream) {
  sample_kernel<<<dim3(a.nchunk, units), kNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_debug_philox(uint64_t seed, int b, int h, int grp, int j0, int n,
                               uint32_t* words, hipStream_t stream) {
  debug_philox_kernel<<<(n + 255) / 256, 256, 0, stream>>>(seed, b, h, grp, j0, n, words);
  return hipGetLastError();
}

hipError_t launch_debug_sexp(const float* x, float* y, int n, hipStream_t stream) {
  debug_sexp_kernel<<<(n + 255) / 256, 256, 0, stream>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace ssa

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
// u_j < m w_j / W_lb up to a margin that covers every rounding, with
// W_lb <= W (1 - 2^-10) a lower bound of the normaliser taken from the
// first-digit histogram (u_j W_lb <= u_j W, so no token that the exact test
// would include is dropped; the filter states the bound).  The final sample
// pass only visits these lists.
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
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b, a.max_topk, a.kmult);
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
  __shared__ int dig_sh[4];  // the digit's bin, remainder, mode and count above
  __shared__ unsigned long long dig_m;
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
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b, a.max_topk, a.kmult);
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
  // The digit is searched by one wave; the others wait at the barrier.
  if (threadIdx.x < 64) {
    DigitBound d{kBins, 0, 0ull, 0};
    int above = 0;
    if (p.k_eff > 0) {
      int bc, rc;  // where the count bound ends (its rank search)
      wave_find_bin<int>(hist, kBins, p.k_eff, &bc, &rc);
      d = DigitBound{bc, rc, 0ull, kBoundCount};
      if (topp) {
        unsigned long long qs = 0ull;
        for (int i = threadIdx.x; i < kBins; i += 64) qs += mh[i];
        const unsigned long long tau = mass_target(p.p, wave_sum(qs));
        if (tau == 0ull) {
          d = DigitBound{kBins, 0, 0ull, 0};
        } else {
          int bm;
          unsigned long long rm;
          wave_find_bin<unsigned long long>(mh, kBins, tau, &bm, &rm);
          d = combine_bounds(kBoundCount | kBoundMass, bc, rc, bm, rm);
        }
      }
      // Tokens above the digit: the rank search already counted them when it
      // chose the digit.
      above = d.bin == kBins ? 0
              : (d.bin == bc && (d.mode & kBoundCount)) ? p.k_eff - rc
                                                        : wave_count_above(hist, kBins, d.bin);
    }
    if (threadIdx.x == 0) {
      dig_sh[0] = d.bin;
      dig_sh[1] = d.rem;
      dig_sh[2] = d.mode;
      dig_sh[3] = above;
      dig_m = d.rem_mass;
    }
  }
  __syncthreads();
  const int b1 = dig_sh[0];
  const float M = key_to_float(maxkey);
  double lb = 0.0;
  for (int bin = threadIdx.x; bin < b1; bin += kNT) {
    const uint32_t n = hist[bin];
    const float lo = key_to_float((uint32_t)bin << kDigit1Shift);
    if (n && lo == lo) lb += (double)n * (double)sexp(lo - M);
  }
  lb = block_sum_f64<kNT>(lb, dscr);
  // An injected W gets the same margin, so the filter's test stays necessary
  // for the final test with that W.
  float wlb = (float)(lb * (1.0 - 0x1.0p-10));
  if (a.w_in) wlb = fminf(wlb, (float)((double)a.w_in[u] * (1.0 - 0x1.0p-10)));
  if (threadIdx.x == 0)
    a.thresh[u] = Thresh1{b1, dig_sh[1], wlb, dig_sh[2], dig_m, dig_sh[3], 0};
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
  __shared__ uint32_t stage[kNT / 64][kStage];  // each wave's second-pass entries

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
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b, a.max_topk, a.kmult);
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
  filter_chunk(a, p, t1, M, u, b, h, ui.grp, c, s4, sh, scan_scr, dscr, stage[threadIdx.x >> 6]);
}

// ------------------------------------------------------------------ resolve
// One workgroup per unit: finish the radix select on the candidates (second
// digit from the histogram, third digit from an LDS histogram of the
// candidates sharing the first two digits), then the per-chunk tie counts,
// the tie quota offsets and the tail normaliser W.
//
// Wave w serves the unit's chunks w, w + 16, w + 32, ...; in each, lane l
// takes candidates l, l + 64, ..., so every load reads 256 contiguous bytes
// of a chunk's segment.  The first 64 candidates of the wave's first 16
// chunks stay in registers between the passes (at 50x sparsity a chunk holds
// about 40); the rest are read again in each pass.  The digit searches and
// the scan over the chunks run in one wave between two barriers, and the
// per-chunk counts are wave ballots, so no pass needs an LDS atomic but the
// third-digit histogram's.  Every thread's items are fixed by the chunk
// count, so every sum has a fixed order.
constexpr int kRT = 1024;
constexpr int kRW = kRT / 64;
constexpr int kRSlots = 16;  // chunks per wave whose first 64 candidates stay in registers
constexpr int kMaxResolveChunks = SSA_MAX_SEQ_LEN / kChunk;
static_assert(kBins % kRT == 0, "each resolve thread loads kBins / kRT histogram entries");
static_assert(kRSlots <= 64, "one lane per slot holds the slot's candidate count");

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

// One radix digit of the stratum's end, searched by one wave over the LDS
// count (and, with the mass bound open, mass) histograms: where the open
// bounds end (the one reached first decides) and how many candidates lie
// above that bin.
__device__ __forceinline__ void wave_digit(const uint32_t* hist, const unsigned long long* mh,
                                           int nbins, int mode, int rem,
                                           unsigned long long rem_mass, DigitBound* d,
                                           int* above) {
  int bc = 0, rc = 0, bm = 0;
  unsigned long long rm = 0ull;
  if (mode & kBoundCount) wave_find_bin<int>(hist, nbins, rem, &bc, &rc);
  if (mode & kBoundMass) wave_find_bin<unsigned long long>(mh, nbins, rem_mass, &bm, &rm);
  *d = combine_bounds(mode, bc, rc, bm, rm);
  *above = ((d->mode & kBoundCount) && d->bin == bc) ? rem - rc
                                                     : wave_count_above(hist, nbins, d->bin);
}

__global__ __launch_bounds__(kRT) void resolve_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ unsigned long long mh[kBins];  // mass units per digit (top-p)
  __shared__ int ties_sh[kMaxResolveChunks];  // ties + (candidates above the key << 16)
  __shared__ int dig_sh[4];                   // a digit's bin, remainder, mode, count above
  __shared__ unsigned long long dig_m;        // and its mass remainder
  __shared__ int scan_scr[kRW];
  __shared__ double dscr[kRW];

  const int u = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // The loads that need no sequence parameter come first: the first-digit
  // threshold and the maximum, the second-digit histogram, the wave's chunk
  // counts (lane j: slot j), the first 64 candidate keys and weights of its
  // chunks (read whole within each chunk's segment, from a chunk clamped into
  // the launch's range; entries past a count are never used) and the chunk
  // tail sums.
  constexpr int kHist = kBins / kRT;
  const Thresh1 t1 = a.thresh[u];
  const uint32_t maxkey = a.maxkey[u];
  uint32_t hv[kHist];
#pragma unroll
  for (int j = 0; j < kHist; ++j) hv[j] = a.hist2[(size_t)u * kBins + threadIdx.x + j * kRT];
  const size_t cu = (size_t)u * a.nchunk;
  const uint32_t* ckeys = a.cand_key + (size_t)u * a.seg_ld;
  const float* cws = a.cand_w + (size_t)u * a.seg_ld;
  const int last = a.nchunk - 1;
  const int cnt_l = a.cand_cnt[cu + min(wave + kRW * min(lane, kRSlots - 1), last)];
  uint32_t kr[kRSlots];
  float wr[kRSlots];  // the candidates' tail weights, computed by the filter
#pragma unroll
  for (int j = 0; j < kRSlots; ++j) {
    const size_t at = (size_t)min(wave + kRW * j, last) * kChunk + lane;
    kr[j] = ckeys[at];
    wr[j] = cws[at];
  }
  // This thread's chunk tail sum, with the first loads when every chunk has
  // its own thread (entries past the sequence's chunks are ignored).
  const double wp = a.wpart[cu + min((int)threadIdx.x, last)];
  // The scalar loads of the sequence's parameters go out after these (a
  // scheduling barrier), so their dependent round trips overlap the vector
  // loads in flight, and the vector loads stay here instead of sinking into
  // the branch that uses them.
  __builtin_amdgcn_sched_barrier(0);
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const SeqParams p = seq_params(ui.L, a.topk, a.top_p, a.sample_budget, b, a.max_topk, a.kmult);
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
      const int nc = (p.L + kChunk - 1) / kChunk;  // at most a.nchunk
      double acc = (int)threadIdx.x < nc ? wp : 0.0;
      for (int c = threadIdx.x + kRT; c < nc; c += kRT) acc += a.wpart[cu + c];
      double cs = 0.0;  // this thread's candidates below the threshold key
      int total_ties = 0;  // wave 0 only
      if (t1.mode == 0) {
        st.flags = kFlagNoTopk;
        st.k_eff = 0;
      } else {
#pragma unroll
        for (int j = 0; j < kHist; ++j) hist[threadIdx.x + j * kRT] = hv[j];
        if (t1.mode & kBoundMass)
          for (int i = threadIdx.x; i < kBins; i += kRT) mh[i] = a.hist2m[(size_t)u * kBins + i];
        __syncthreads();
        // Second digit.
        if (wave == 0) {
          DigitBound d;
          int above;
          wave_digit(hist, mh, kBins, t1.mode, t1.rem, t1.rem_mass, &d, &above);
          if (lane == 0) {
            dig_sh[0] = d.bin;
            dig_sh[1] = d.rem;
            dig_sh[2] = d.mode;
            dig_sh[3] = above;
            dig_m = d.rem_mass;
          }
        }
        __syncthreads();
        const DigitBound d2{dig_sh[0], dig_sh[1], dig_m, dig_sh[2]};
        const int above2 = dig_sh[3];
        const bool mass3 = d2.mode & kBoundMass;
        const uint32_t prefix = ((uint32_t)t1.b1 << 11) | (uint32_t)d2.bin;
        for (int i = threadIdx.x; i < kBins3; i += kRT) {
          hist[i] = 0u;
          if (mass3) mh[i] = 0ull;
        }
        __syncthreads();
        // Third digit: LDS histograms of the candidates that share the prefix.
        auto add3 = [&](uint32_t key, float w) {
          if ((key >> kDigit2Shift) == prefix) {
            atomicAdd(&hist[key & (kBins3 - 1)], 1u);
            if (mass3) atomicAdd(&mh[key & (kBins3 - 1)], mass_units(w));
          }
        };
#pragma unroll
        for (int j = 0; j < kRSlots; ++j) {
          const int c = wave + kRW * j;
          if (c < nc) {  // uniform over the wave
            const int n = clamp_count(__builtin_amdgcn_readlane(cnt_l, j), kChunk);
            if (lane < n) add3(kr[j], wr[j]);
            for (int i = lane + 64; i < n; i += 64) add3(ckeys[(size_t)c * kChunk + i],
                                                          cws[(size_t)c * kChunk + i]);
          }
        }
        for (int c = wave + kRW * kRSlots; c < nc; c += kRW) {
          const int n = clamp_count(a.cand_cnt[cu + c], kChunk);
          for (int i = lane; i < n; i += 64) add3(ckeys[(size_t)c * kChunk + i],
                                                   cws[(size_t)c * kChunk + i]);
        }
        __syncthreads();
        if (wave == 0) {
          DigitBound d;
          int above;
          wave_digit(hist, mh, kBins3, d2.mode, d2.rem, d2.rem_mass, &d, &above);
          if (lane == 0) {
            dig_sh[0] = d.bin;
            dig_sh[1] = d.rem;
            dig_sh[2] = d.mode;
            dig_sh[3] = above;
            dig_m = d.rem_mass;
          }
        }
        __syncthreads();
        const DigitBound d3{dig_sh[0], dig_sh[1], dig_m, dig_sh[2]};
        const int above3 = dig_sh[3];
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
        // Ties on the threshold key per chunk and, for early stopping, the
        // candidates above it (wave ballots; packed as ties + (above << 16),
        // each at most 4096), and the weight of the candidates strictly below
        // it (each thread over its fixed items, in order; summed with the
        // chunk sums below).
        const uint32_t tkey = st.tkey;
        const bool want_above = a.stop_off != nullptr;  // only early stopping uses them
        auto count = [&](uint32_t key, float w, bool v, int& packed) {
          packed += __popcll(__ballot(v && key == tkey));
          if (want_above) packed += __popcll(__ballot(v && key > tkey)) << 16;
          if (v && key < tkey) cs += (double)w;
        };
#pragma unroll
        for (int j = 0; j < kRSlots; ++j) {
          const int c = wave + kRW * j;
          if (c < nc) {  // uniform over the wave
            const int n = clamp_count(__builtin_amdgcn_readlane(cnt_l, j), kChunk);
            int packed = 0;
            count(kr[j], wr[j], lane < n, packed);
            for (int i0 = 64; i0 < n; i0 += 64) {
              const int i = i0 + lane;
              const size_t at = (size_t)c * kChunk + min(i, kChunk - 1);
              count(ckeys[at], cws[at], i < n, packed);
            }
            if (lane == 0) ties_sh[c] = packed;
          }
        }
        for (int c = wave + kRW * kRSlots; c < nc; c += kRW) {
          const int n = clamp_count(a.cand_cnt[cu + c], kChunk);
          int packed = 0;
          for (int i0 = 0; i0 < n; i0 += 64) {
            const int i = i0 + lane;
            const size_t at = (size_t)c * kChunk + min(i, kChunk - 1);
            count(ckeys[at], cws[at], i < n, packed);
          }
          if (lane == 0) ties_sh[c] = packed;
        }
        __syncthreads();  // the chunks' tie counts are complete
        if (wave == 0) {
          // Exclusive scan of the tie counts over the chunks, 64 at a time.
          int run = 0;
          for (int c0 = 0; c0 < nc; c0 += 64) {
            const int c = c0 + lane;
            const int v = c < nc ? ties_sh[c] & 0xffff : 0;
            const int inc = wave_inclusive_scan<int>(v);
            if (c < nc) {
              a.ties_before[cu + c] = run + inc - v;
              a.tiecnt[cu + c] = v;
            }
            run += __builtin_amdgcn_readlane(inc, 63);
          }
          total_ties = run;
        }
        if (a.stop_off) stop_offsets(a, u, cu, nc, ties_sh, scan_scr);
      }
      W = block_sum_f64<kRT>(acc + cs, dscr);  // every thread's share, one fixed tree
      // The ties beyond the quota are tail tokens (wave 0 holds their count;
      // only thread 0 writes W).
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
  if (a.w64 && threadIdx.x == 0) a.w64[u] = W;
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
// methodology parts 2 and 3.  The deterministic stratum, in its order (key
// descending, position ascending), is visited in 64-token blocks while the
// online-softmax state of every query row of the unit (each query head of each
// member of its query group) takes in the block's exact attention mass; the
// visit stops after the first block at which every row's gain in its softmax
// denominator l is 0 or below tau times the row's l so far.  Gains are counted
// in integer units floor(2^38 sexp(l - M_row)) of exact logits computed in a
// specified float32 order, so the cut is exact and reproducible.  A token's
// word is ((~key) << 32) | position, so ascending words are the stratum's
// order, and the cut is published as the last word kept: the sample kernel
// drops every deterministic token whose word is larger.  The stratum is the
// tokens above the threshold key T followed by the first ties on T (ranked by
// position); only the former need sorting.  Seven kernels, none with a
// global atomic:
//   stop_gather: each chunk writes its words above T (its listed tokens above
//     the threshold digit, then its candidates above T) at the offset the
//     resolve kernel computed for it, and its ties within the quota straight
//     to their ranks (after every word above T);
//   stop_sort: one workgroup sorts each 1024-word slice (4 words per thread
//     in registers, cross-wave exchanges through LDS);
//   stop_pair: for every pair of slices, the number of words of one below
//     each word of the other (searched in LDS), one count array per pair;
//   stop_final: each word's rank = its index in its slice + those counts;
//     the words stored in rank order;
//   stop_logit: one wave per 64-token block of the order computes every
//     row's exact logit of its tokens (key rows through the block table)
//     and the block's maximum of each row;
//   stop_gain: one wave per block sums its tokens' units for every row;
//   stop_cut: one workgroup per unit takes the block gains' prefix sums
//     and the first block where every row agrees, and writes the last word
//     kept.
constexpr int kStopBlock = 64;
constexpr int kStopMax = SSA_STOP_MAX_STRATUM;  // largest stratum that is ordered
constexpr int kStopRows = SSA_STOP_MAX_ROWS;    // query rows per unit, at most
constexpr int kSlice = 1024;     // words sorted per workgroup
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
  const unsigned __int128 rhs = (unsigned __int128)mant * acc;          // < 2^88
  const int D = 24 - e;                                                 // >= 24
  if (gain == 0ull) return rhs != 0;
  if (D >= 88 || (64 - __builtin_clzll(gain)) + D > 127) return false;  // lhs >= 2^88 > rhs
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
  const int tie0 = a.ties_before[ci];  // ties on T in earlier chunks
  const int nvalid = min(kChunk, st.L - c0);
  const float* srow = a.scores + (size_t)u * a.score_ld;
  unsigned long long* out = a.stop_words + (size_t)u * kStopMax;
  unsigned long long* rword = a.stop_rword + (size_t)u * kStopMax;
  for (int i = threadIdx.x; i < n_above; i += kNT) {
    const int pos = c0 + min(max(a.list_idx[seg + i] - c0, 0), nvalid - 1);
    const int at = off + i;
    if (at >= 0 && at < n_words) out[at] = stratum_word(order_key(srow[pos]), pos);
  }
  // Candidates above T, compacted in list (position) order, and the ties on
  // T within the quota, at ranks n_words + (their rank among the ties).
  int run = off + n_above;
  int tie_run = tie0;
  for (int base = 0; base < ncand; base += kNT) {
    const int i = base + threadIdx.x;
    const uint32_t key = i < ncand ? a.cand_key[seg + i] : 0u;
    const bool in = i < ncand && key > st.tkey;
    const bool tie = i < ncand && key == st.tkey;
    int tot;
    const int ex = block_exclusive_scan<kNT>((in ? 1 : 0) | (tie ? 0x10000 : 0), scan_scr, &tot);
    const int pos = c0 + min(max((i < ncand ? a.cand_idx[seg + i] : c0) - c0, 0), nvalid - 1);
    const int at = run + (ex & 0xffff);
    if (in && at >= 0 && at < n_words) out[at] = stratum_word(key, pos);
    const int tr = tie_run + (ex >> 16);
    if (tie && tr >= 0 && tr < st.ties_needed) {
      const int rank = n_words + tr;
      if (rank < kStopMax) rword[rank] = stratum_word(key, pos);
    }
    run += tot & 0xffff;
    tie_run += tot >> 16;
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
  unsigned long long* rword = a.stop_rword + (size_t)u * kStopMax;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // words are distinct, so ranks are: a permutation of [0, n_words)
    if (x[e] != ~0ull && rank[e] < n_words) rword[rank[e]] = x[e];
  }
}

// The exact logit of each (rank, query row) of a unit's stratum, in the
// specified float32 order: lane c of a token's D/8 lanes holds its 8-dim
// slice c, sums the 8 exact bf16 products in dim order, and the slices are
// combined pairwise by butterfly exchanges (every lane of the token ends with
// the same sum); then one multiply by the softmax scale.  Rows whose member's
// span excludes the token get -inf.  The block's largest order key of each
// row goes to stop_mkey (0: none).  Grid: (kStopMax / 64, units) x 256
// threads: wave w takes the block's tokens 16 w .. 16 w + 15, resolves them
// to cache rows in one round of loads and loads all their key slices
// together.
constexpr int kLogitT = 256;
constexpr int kLogitTok = kStopBlock / (kLogitT / 64);  // tokens per wave
template <int D, bool SPLIT>
__global__ __launch_bounds__(kLogitT) void stop_logit_kernel(SelectArgs a) {
  constexpr int LPT = D / 8;           // lanes per token
  constexpr int TPI = 64 / LPT;        // tokens per step
  constexpr int NIT = kLogitTok / TPI;  // steps per wave
  static_assert(kStopRows * LPT <= kLogitT, "one 16-byte query slice per thread");
  __shared__ float qsh[kStopRows * D];
  __shared__ uint32_t row_sh[kStopBlock];
  __shared__ int pos_sh[kStopBlock];
  __shared__ uint32_t mk_sh[kLogitT / 64][kStopRows];
  const int u = blockIdx.y;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  if (!stop_applies(st)) return;  // uniform
  const int n = min(st.k_eff, kStopMax);
  const int r0 = blockIdx.x * kStopBlock;
  if (r0 >= n) return;  // uniform
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const int h = ui.h;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int t0 = ui.grp * a.g;                 // the group's first member
  const int nmem = min(a.g, a.T - t0);
  const int rows = min(nmem * a.G, kStopRows);  // the host guarantees nmem * G <= kStopRows
  const int P = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int L = ui.L;
  if (lane < kLogitTok) {
    // Token j of the block (rank r0 + j < kStopMax: the load stays in the
    // unit's word array; ranks past the stratum are masked below).
    const int j = wave * kLogitTok + lane;
    const unsigned long long w = a.stop_rword[(size_t)u * kStopMax + r0 + j];
    const int pos = min(max((int)(uint32_t)w, 0), max(L - 1, 0));
    int blk = a.block_table[(size_t)b * a.max_blocks + (pos >> 4)];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    row_sh[j] = (uint32_t)((blk * a.Hkv + h) * kBlockTokens + (pos & 15));
    pos_sh[j] = pos;
  }
  {
    // The query rows in LDS as floats: thread (r, c) stages slice c of row r.
    const int r = tid / LPT;
    const int c = tid - r * LPT;
    if (r < rows) {
      const int t = t0 + r / a.G;
      const uint4 v = *reinterpret_cast<const uint4*>(
          a.q + ((size_t)(b * a.T + t) * a.Hq + h * a.G + r % a.G) * D + c * 8);
      float* dst = qsh + r * D + c * 8;
      dst[0] = bf16_lo(v.x);
      dst[1] = bf16_hi(v.x);
      dst[2] = bf16_lo(v.y);
      dst[3] = bf16_hi(v.y);
      dst[4] = bf16_lo(v.z);
      dst[5] = bf16_hi(v.z);
      dst[6] = bf16_lo(v.w);
      dst[7] = bf16_hi(v.w);
    }
  }
  __syncthreads();
  const int sl = lane % LPT;  // this lane's slice
  const int tk = lane / LPT;
  // This lane's key slice: dims sl*8 .. +8 of row r are at kb + r * kld.
  const uint16_t* kb;
  uint32_t kld;
  {
    const int dim = sl * 8;
    if (!SPLIT) {
      kb = a.k_cache + dim;
      kld = D;
    } else {
      const int lo = 2 * a.pair_begin;
      const int nd = 2 * a.pair_count;
      const bool scored = dim >= lo && dim < lo + nd;
      kb = scored ? a.k_cache + (dim - lo) : a.k_rest + (dim < lo ? dim : dim - nd);
      kld = scored ? nd : D - nd;
    }
  }
  uint4 kv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    kv[it] = *reinterpret_cast<const uint4*>(
        kb + (size_t)row_sh[wave * kLogitTok + it * TPI + tk] * kld);
  float* out = a.stop_logit + (size_t)u * kStopMax * kStopRows;
  // One query row at a time (a uniform runtime loop), the wave's tokens
  // unrolled inside it, so every key slice stays in a fixed register.
  for (int r = 0; r < rows; ++r) {
    float qr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qr[i] = qsh[r * D + sl * 8 + i];
    const int span = member_span(P, a.T, t0 + r / a.G);
    uint32_t mk = 0u;  // this lane's largest order key of the row
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int j = wave * kLogitTok + it * TPI + tk;  // the token's index in the block
      const int rank = r0 + j;
      const float kf[8] = {bf16_lo(kv[it].x), bf16_hi(kv[it].x), bf16_lo(kv[it].y),
                           bf16_hi(kv[it].y), bf16_lo(kv[it].z), bf16_hi(kv[it].z),
                           bf16_lo(kv[it].w), bf16_hi(kv[it].w)};
      float acc = qr[0] * kf[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) acc = acc + qr[i] * kf[i];  // exact products
      const float l = butterfly<LPT>(acc) * a.scale;
      const bool valid = rank < n;
      const bool vis = pos_sh[j] < span;
      if (valid && sl == r % LPT) out[(size_t)rank * kStopRows + r] = vis ? l : -INFINITY;
      const uint32_t k = (valid && vis && l > -INFINITY) ? order_key(l) : 0u;
      mk = k > mk ? k : mk;
    }
    const uint32_t v = wave_max_u32(mk);
    if (lane == 0) mk_sh[wave][r] = v;
  }
  __syncthreads();
  if (tid < rows) {
    uint32_t v = mk_sh[0][tid];
#pragma unroll
    for (int w = 1; w < kLogitT / 64; ++w) v = mk_sh[w][tid] > v ? mk_sh[w][tid] : v;
    a.stop_mkey[((size_t)u * (kStopMax / kStopBlock) + blockIdx.x) * kStopRows + tid] = v;
  }
}

// Gains of the 64-token blocks of the order: block i's gain for row r is the
// sum over its tokens of floor(2^38 sexp(l - M_r)), M_r the row's largest
// logit over the stratum (the maximum of the blocks' maxima; -inf entries
// add nothing).  Grid: (kStopMax / 64, units) x 64 threads, lane = token;
// the blocks' maxima and the lane's row logits are loaded together.
__global__ __launch_bounds__(64) void stop_gain_kernel(SelectArgs a) {
  constexpr int kNB = kStopMax / kStopBlock;
  const int u = blockIdx.y;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  if (!stop_applies(st)) return;  // uniform
  const int n = min(st.k_eff, kStopMax);
  const int nb = (n + kStopBlock - 1) / kStopBlock;
  const int i = blockIdx.x;
  if (i >= nb) return;  // uniform
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int rows = min(min(a.g, a.T - ui.grp * a.g) * a.G, kStopRows);
  const int lane = threadIdx.x;
  const int rank = i * kStopBlock + lane;  // < kStopMax
  const float4* lg4 =
      reinterpret_cast<const float4*>(a.stop_logit + ((size_t)u * kStopMax + rank) * kStopRows);
  float l[kStopRows];
#pragma unroll
  for (int k = 0; k < kStopRows / 4; ++k) {
    const float4 v = lg4[k];
    l[4 * k] = v.x;
    l[4 * k + 1] = v.y;
    l[4 * k + 2] = v.z;
    l[4 * k + 3] = v.w;
  }
  // This lane's blocks lane, lane + 64, ...: their maxima of every row, the
  // blocks past nb (not written by this call) counting as none.
  uint32_t m[kStopRows];
#pragma unroll
  for (int r = 0; r < kStopRows; ++r) m[r] = 0u;
  const uint4* mkb = reinterpret_cast<const uint4*>(a.stop_mkey + (size_t)u * kNB * kStopRows);
#pragma unroll
  for (int k = 0; k < kNB / 64; ++k) {
    const int blk = lane + 64 * k;
    uint4 v[kStopRows / 4];
#pragma unroll
    for (int c = 0; c < kStopRows / 4; ++c) v[c] = mkb[blk * (kStopRows / 4) + c];
    if (blk < nb) {
#pragma unroll
      for (int c = 0; c < kStopRows / 4; ++c) {
        m[4 * c] = v[c].x > m[4 * c] ? v[c].x : m[4 * c];
        m[4 * c + 1] = v[c].y > m[4 * c + 1] ? v[c].y : m[4 * c + 1];
        m[4 * c + 2] = v[c].z > m[4 * c + 2] ? v[c].z : m[4 * c + 2];
        m[4 * c + 3] = v[c].w > m[4 * c + 3] ? v[c].w : m[4 * c + 3];
      }
    }
  }
  unsigned long long* gout = a.stop_gain + ((size_t)u * kNB + i) * kStopRows;
#pragma unroll
  for (int r = 0; r < kStopRows; ++r) {
    if (r >= rows) break;  // uniform
    const uint32_t mk = wave_max_u32(m[r]);
    const unsigned long long q = (rank < n && l[r] > -INFINITY && mk)
                                     ? mass_units(sexp(l[r] - key_to_float(mk)))
                                     : 0ull;
    const unsigned long long g = wave_sum(q);
    if (lane == 0) gout[r] = g;
  }
}

// Grid: units x kCutT threads.  Per row, the mass so far after each block
// (prefix sums of the block gains); block i agrees when every row's gain is
// 0 or below tau times its mass so far; the cut follows the first block
// that agrees.
constexpr int kCutT = 256;
constexpr int kCutW = kCutT / 64;
static_assert(kCutT == kStopMax / kStopBlock, "one thread per block of the order");
__global__ __launch_bounds__(kCutT) void stop_cut_kernel(SelectArgs a) {
  __shared__ unsigned long long scan_m[kCutW];
  __shared__ int first_sh;
  const int u = blockIdx.x;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  const int tid = threadIdx.x;
  if (!stop_applies(st)) {  // uniform
    if (tid == 0) a.stop_cut[u] = ~0ull;
    return;
  }
  const int n = min(st.k_eff, kStopMax);
  const int nb = (n + kStopBlock - 1) / kStopBlock;
  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int rows = min(min(a.g, a.T - ui.grp * a.g) * a.G, kStopRows);
  // Thread tid holds block tid's gains (all 16 words loaded together; blocks
  // at or past nb were not written and are ignored).
  unsigned long long g[kStopRows];
  {
    const ulonglong2* gp = reinterpret_cast<const ulonglong2*>(
        a.stop_gain + ((size_t)u * kCutT + tid) * kStopRows);
#pragma unroll
    for (int k = 0; k < kStopRows / 2; ++k) {
      const ulonglong2 v = gp[k];
      g[2 * k] = tid < nb ? v.x : 0ull;
      g[2 * k + 1] = tid < nb ? v.y : 0ull;
    }
  }
  if (tid == 0) first_sh = 0x7fffffff;
  bool agree = tid < nb;
#pragma unroll
  for (int r = 0; r < kStopRows; ++r) {
    if (r >= rows) break;  // uniform
    unsigned long long tot;
    const unsigned long long acc = block_exclusive_scan<kCutT>(g[r], scan_m, &tot) + g[r];
    if (g[r] != 0ull && !gain_below(g[r], acc, a.stop_tau)) agree = false;
  }
  __syncthreads();
  if (agree) atomicMin(&first_sh, tid);
  __syncthreads();
  const int kept = first_sh == 0x7fffffff ? n : min(n, (first_sh + 1) * kStopBlock);
  if (tid == 0)
    a.stop_cut[u] = kept < n ? a.stop_rword[(size_t)u * kStopMax + kept - 1] : ~0ull;
}

// ------------------------------------------------------------------ sample
// Per chunk: membership of the listed tokens only -- above-threshold tokens
// and candidates above the threshold key (or within the tie quota) form the
// deterministic set; the other candidates and the listed sampling candidates
// take the exact inclusion test with the final W.  Membership is kept in two
// LDS bitmaps (deterministic, sampled) with each sampled token's logit bias
// -log(pi) beside them, and the chunk's segment is written from the bitmaps:
// deterministic tokens ascending, then sampled tokens ascending.  With
// emit_rows the segment holds cache row numbers (for the fused attention
// stage) instead of positions.
constexpr int kMapWords = kChunk / 32;

__device__ __forceinline__ void sample_one(const UnitState& st, uint64_t seed, int b, int h,
                                           int grp, int t, float w, int c0, int nvalid,
                                           uint32_t* rbits, float* bias) {
  if ((unsigned)(t - c0) >= (unsigned)nvalid) return;  // not a position of this chunk
  const uint4 wd = philox_block(seed, b, h, (uint32_t)t >> 2, grp);
  const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
  const float mw = (float)st.m * w;
  if (uniform24(words[t & 3]) * st.W < mw) {
    const int i = t - c0;
    bias[i] = -logf(fminf(1.0f, mw / st.W));
    atomicOr(&rbits[i >> 5], 1u << (i & 31));
  }
}

__device__ __forceinline__ void mark_det(uint32_t* sbits, int i) {
  atomicOr(&sbits[i >> 5], 1u << (i & 31));
}

__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(8))) void sample_kernel(
    SelectArgs a) {
  __shared__ uint32_t sbits[kMapWords];  // deterministic positions of the chunk
  __shared__ uint32_t rbits[kMapWords];  // sampled positions
  __shared__ float bias[kChunk];         // a sampled position's -log(pi)
  __shared__ int scan_scr[kNT / 64];
  static_assert(kPer == kBlockTokens, "a thread's positions are one cache block");
  static_assert(kPer == 16 && kMapWords * 2 == kNT, "a thread's positions are half a bitmap word");

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
  const float* cw = a.cand_w + (size_t)u * a.seg_ld + c0;
  const int l_first = lidx[tid];
  const float w_first = lw[tid];
  const int c_first = cidx[tid];
  const uint32_t k_first = ckey[tid];
  const float cw_first = cw[tid];
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  // Counts are clamped to the segment and positions checked against the
  // chunk, so no value in the workspace can address outside it.
  const int n_above = clamp_count(a.list_cnt[2 * ci], kChunk);
  const int n_samp = clamp_count(a.list_cnt[2 * ci + 1], kChunk - n_above);
  const int ncand = clamp_count(a.cand_cnt[ci], kChunk);
  const int before = a.ties_before[ci];
  const int ties_here = a.tiecnt[ci];
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
  {
    // Dense units take every valid position; otherwise the maps start empty.
    const int wi = tid & (kMapWords - 1);
    const int lo = wi * 32;
    const uint32_t full = nvalid >= lo + 32 ? ~0u : (nvalid <= lo ? 0u : (1u << (nvalid - lo)) - 1u);
    if (tid < kMapWords)
      sbits[wi] = dense ? full : 0u;
    else
      rbits[wi] = 0u;
  }
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
          mark_det(sbits, t - c0);
      } else {
        sample_one(st, seed, b, h, ui.grp, t, i == tid ? w_first : lw[i], c0, nvalid, rbits,
                   bias);
      }
    }
    if (!(st.flags & kFlagNoTopk)) {
      // Threshold-digit candidates, in index order: key above T -> S; key == T
      // -> S while the tie quota lasts; otherwise a tail token, whose weight
      // the filter stored.  Ties are ranked by a block scan only in chunks
      // that hold one (the resolve counted them).
      int run = 0;  // ties seen in earlier rounds of this loop
      for (int base = 0; base < ncand; base += kNT) {
        const int i = base + tid;
        const bool v = i < ncand;
        const uint32_t key = v ? (base == 0 ? k_first : ckey[i]) : 0u;
        const int t = v ? (base == 0 ? c_first : cidx[i]) : 0;
        const bool tie = v && key == st.tkey;
        int rank = 0;
        if (ties_here != 0) {  // uniform over the workgroup
          int tot;
          rank = before + run + block_exclusive_scan<kNT>(tie ? 1 : 0, scan_scr, &tot);
          run += tot;
        }
        if (v) {
          if (key > st.tkey || (tie && rank < st.ties_needed)) {
            // stratum tokens past the early stop are neither read nor sampled
            if ((unsigned)(t - c0) < (unsigned)nvalid && stratum_word(key, t) <= cut)
              mark_det(sbits, t - c0);
          } else if (sampling) {
            sample_one(st, seed, b, h, ui.grp, t, base == 0 ? cw_first : cw[i], c0, nvalid,
                       rbits, bias);
          }
        }
      }
    }
  }
  __syncthreads();
  // Compaction from the bitmaps: the thread's 16 consecutive positions are
  // half of one word of each map.
  const int tb = threadIdx.x * kPer;
  const int sh16 = (tid & 1) * 16;
  const uint32_t smask = (sbits[tid >> 1] >> sh16) & 0xffffu;
  const uint32_t rmask = (rbits[tid >> 1] >> sh16) & 0xffffu & ~smask;
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
  // Ascending bits keep both lists in index order.
  for (uint32_t rest = smask | rmask; rest != 0u; rest &= rest - 1u) {
    const int i = __builtin_ctz(rest);
    const int t = c0 + tb + i;
    const int v = a.emit_rows ? (blk * a.Hkv + h) * kBlockTokens + (t & 15) : t;
    if ((smask >> i) & 1u) {
      sidx[ws] = v;
      slw[ws] = 0.0f;
      ++ws;
    } else {
      sidx[wr] = v;
      slw[wr] = bias[tb + i];
      ++wr;
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
  // The filter's variant (the key is a kernel argument, uniform); the sample
  // kernel's generic one decides every final inclusion the parity tests check.
  const uint4 wd = philox_block_uniform_key(seed, b, h, j >> 2, grp);
  const uint32_t w4[4] = {wd.x, wd.y, wd.z, wd.w};
  words[i] = w4[j & 3u];
}

__global__ void debug_sexp_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = sexp(x[i]);
}

__global__ void debug_tail_exp_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = tail_exp(x[i]);
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
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  stop_gather_kernel<<<dim3(a.nchunk, units), kNT, 0, stream>>>(a);
  stop_sort_kernel<<<dim3(kSlices, units), kSortT, 0, stream>>>(a);
  stop_pair_kernel<<<dim3(kSlices * kSlices, units), kNT, 0, stream>>>(a);
  stop_final_kernel<<<dim3(kSlices, units), kNT, 0, stream>>>(a);
  const dim3 lg(kStopMax / kStopBlock, units);
  const bool split = a.k_rest != nullptr;
  if (a.d == 128 && !split)
    stop_logit_kernel<128, false><<<lg, kLogitT, 0, stream>>>(a);
  else if (a.d == 128)
    stop_logit_kernel<128, true><<<lg, kLogitT, 0, stream>>>(a);
  else if (!split)
    stop_logit_kernel<64, false><<<lg, kLogitT, 0, stream>>>(a);
  else
    stop_logit_kernel<64, true><<<lg, kLogitT, 0, stream>>>(a);
  stop_gain_kernel<<<lg, 64, 0, stream>>>(a);
  stop_cut_kernel<<<units, kCutT, 0, stream>>>(a);
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

hipError_t launch_debug_tail_exp(const float* x, float* y, int n, hipStream_t stream) {
  debug_tail_exp_kernel<<<(n + 255) / 256, 256, 0, stream>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace ssa

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
//   tail:   w_j = sexp(s_j - M), W = sum over the tail, computed directly in
//           fp64 (never as total minus top-k, which cancels);
//   sample: include j iff fl(u_j * W) < fl(m * w_j), u_j from Philox4x32-10
//           keyed by the sequence's seed with counter (j >> 2, h, b, 0);
//           pi_j = min(1, fl(m * w_j) / W); the logit bias is -log(pi_j).
//
// A sequence is processed in 4096-token chunks.  Each chunk's selected tokens
// are written to its own segment in index order, so no grid-wide ordering is
// needed and the attention stage splits work along chunk boundaries.  Every
// sum has a fixed order and only integer atomics are used: results are
// bitwise reproducible.
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

constexpr int kNT = 256;             // threads per chunk workgroup
constexpr int kPer = kChunk / kNT;   // 16 consecutive tokens per thread

// Coalesced copy of the chunk's scores into LDS (entries past L are unused).
// All of a thread's loads are issued before the first LDS store.
__device__ __forceinline__ void stage_chunk_scores(const float* srow, int c0, int L, float* sh) {
  float v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int t = c0 + threadIdx.x + k * kNT;
    v[k] = t < L ? srow[t] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) sh[threadIdx.x + k * kNT] = v[k];
  __syncthreads();
}

// ------------------------------------------------------------------ threshold
// First radix digit of the k-th largest key of every unit, from the unit's
// first-digit histogram (one workgroup per unit).
__global__ __launch_bounds__(kNT) void threshold_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ int scan_scr[kNT / 64];
  __shared__ int pair[2];
  const int u = blockIdx.x;
  const int b = u / a.Hkv;
  const SeqParams p = seq_params(a.seq_lens, a.topk, a.sample_budget, b, a.max_seq_len);
  if (p.dense || p.k_eff == 0 || p.L == 0) {
    if (threadIdx.x == 0) a.thresh[u] = Thresh1{kBins, 0};
    return;
  }
  for (int i = threadIdx.x; i < kBins; i += kNT) hist[i] = a.hist1[(size_t)u * kBins + i];
  __syncthreads();
  int b1, rem;
  find_rank_bin<kNT>(hist, kBins, p.k_eff, scan_scr, pair, &b1, &rem);
  if (threadIdx.x == 0) a.thresh[u] = Thresh1{b1, rem};
}

// ------------------------------------------------------------------ filter
// Per chunk: tokens whose first digit is above the unit's threshold digit are
// in the deterministic set; tokens on the threshold digit become candidates
// (written in index order, second-digit histogram updated); tokens below it
// are tail tokens, whose weights are summed here in fp64.
__global__ __launch_bounds__(kNT) void filter_kernel(SelectArgs a) {
  __shared__ float sh[kChunk];
  __shared__ int scan_scr[kNT / 64];
  __shared__ double dscr[kNT / 64];

  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / a.Hkv;
  const SeqParams p = seq_params(a.seq_lens, a.topk, a.sample_budget, b, a.max_seq_len);
  const int c0 = c * kChunk;
  if (c0 >= p.L || p.dense) return;  // uniform over the workgroup
  const int b1 = a.thresh[u].b1;     // 2048 when there is no deterministic set
  const float M = key_to_float(a.maxkey[u]);
  stage_chunk_scores(a.scores + (size_t)u * a.score_ld, c0, p.L, sh);

  const int tb = threadIdx.x * kPer;
  uint32_t candmask = 0u;
  double wsum = 0.0;
  uint32_t keys[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float s = sh[tb + i];
    const uint32_t key = order_key(s);
    keys[i] = key;
    const int bin = (int)(key >> kDigit1Shift);
    if (c0 + tb + i < p.L) {
      if (bin == b1)
        candmask |= 1u << i;
      else if (bin < b1)
        wsum += (double)sexp(s - M);
    }
  }
  int total;
  const int off = block_exclusive_scan<kNT>(__popc(candmask), scan_scr, &total);
  int32_t* cidx = a.cand_idx + (size_t)u * a.seg_ld + c0;
  uint32_t* ckey = a.cand_key + (size_t)u * a.seg_ld + c0;
  int w = off;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (candmask & (1u << i)) {
      cidx[w] = c0 + tb + i;
      ckey[w] = keys[i];
      ++w;
      atomicAdd(&a.hist2[(size_t)u * kBins + ((keys[i] >> kDigit2Shift) & (kBins - 1))], 1u);
    }
  }
  const double wtot = block_sum_f64<kNT>(wsum, dscr);
  if (threadIdx.x == 0) {
    const size_t ci = (size_t)u * a.nchunk + c;
    a.cand_cnt[ci] = total;
    a.wpart[ci] = wtot;
  }
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

// Candidate passes: thread t serves chunk (t / tpc) + k * (kRT / tpc) and,
// inside it, items (t % tpc) + i * tpc.  Every load is independent and every
// thread's items are fixed by (nc, t): sums over them have a fixed order.
__device__ __forceinline__ int threads_per_chunk(int nc) {
  int tpc = kRT;
  while (tpc > 1 && tpc * nc > kRT) tpc >>= 1;
  return tpc;
}

__global__ __launch_bounds__(kRT) void resolve_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ int ties_sh[kMaxResolveChunks];
  __shared__ int scan_scr[kRW];
  __shared__ int pair[2];
  __shared__ double dscr[kRW];

  const int u = blockIdx.x;
  const int b = u / a.Hkv;
  const SeqParams p = seq_params(a.seq_lens, a.topk, a.sample_budget, b, a.max_seq_len);
  UnitState st;
  st.tkey = 0u;
  st.ties_needed = 0;
  st.M = 0.0f;
  st.W = 0.0f;
  st.flags = 0;
  st.k_eff = p.k_eff;
  st.m = p.m;
  st.L = p.L;
  const size_t cu = (size_t)u * a.nchunk;
  const uint32_t* ckeys = a.cand_key + (size_t)u * a.seg_ld;
  double W = 0.0;

  if (p.L == 0) {
    st.flags = kFlagEmpty;
  } else {
    st.M = key_to_float(a.maxkey[u]);
    if (p.dense) {
      st.flags = kFlagDense;
    } else {
      const int nc = (p.L + kChunk - 1) / kChunk;
      const int tpc = threads_per_chunk(nc);
      const int cstep = kRT / tpc;
      const int csub = threadIdx.x % tpc;
      double ctail = 0.0;
      int total_ties = 0;
      if (p.k_eff == 0) {
        st.flags = kFlagNoTopk;
      } else {
        const Thresh1 t1 = a.thresh[u];
        for (int i = threadIdx.x; i < kBins; i += kRT) hist[i] = a.hist2[(size_t)u * kBins + i];
        for (int c = threadIdx.x; c < nc; c += kRT) ties_sh[c] = 0;
        __syncthreads();
        int b2, rem2, b3, rem3;
        find_rank_bin<kRT>(hist, kBins, t1.rem, scan_scr, pair, &b2, &rem2);
        const uint32_t prefix = ((uint32_t)t1.b1 << 11) | (uint32_t)b2;
        for (int i = threadIdx.x; i < kBins3; i += kRT) hist[i] = 0u;
        __syncthreads();
        for (int c = threadIdx.x / tpc; c < nc; c += cstep) {
          const int n = a.cand_cnt[cu + c];
          const uint32_t* ck = ckeys + (size_t)c * kChunk;
#pragma unroll 4
          for (int i = csub; i < n; i += tpc) {
            const uint32_t key = ck[i];
            if ((key >> kDigit2Shift) == prefix) atomicAdd(&hist[key & (kBins3 - 1)], 1u);
          }
        }
        __syncthreads();
        find_rank_bin<kRT>(hist, kBins3, rem2, scan_scr, pair, &b3, &rem3);
        st.tkey = (prefix << kDigit2Shift) | (uint32_t)b3;
        st.ties_needed = rem3;
        // Ties on the threshold key per chunk (integer), and the weight of the
        // candidates strictly below it.
        double cs = 0.0;
        for (int c = threadIdx.x / tpc; c < nc; c += cstep) {
          const int n = a.cand_cnt[cu + c];
          const uint32_t* ck = ckeys + (size_t)c * kChunk;
          int ties = 0;
#pragma unroll 4
          for (int i = csub; i < n; i += tpc) {
            const uint32_t key = ck[i];
            ties += key == st.tkey;
            if (key < st.tkey) cs += (double)sexp(key_to_float(key) - st.M);
          }
          if (ties) atomicAdd(&ties_sh[c], ties);
        }
        ctail = block_sum_f64<kRT>(cs, dscr);
        int run = 0;
        for (int c0 = 0; c0 < nc; c0 += kRT) {
          const int c = c0 + threadIdx.x;
          const int v = c < nc ? ties_sh[c] : 0;
          int tot;
          const int ex = block_exclusive_scan<kRT>(v, scan_scr, &tot);
          if (c < nc) {
            a.ties_before[cu + c] = run + ex;
            a.tiecnt[cu + c] = v;
          }
          run += tot;
        }
        total_ties = run;
      }
      double acc = 0.0;
      for (int c = threadIdx.x; c < nc; c += kRT) acc += a.wpart[cu + c];
      W = block_sum_f64<kRT>(acc, dscr) + ctail;
      if (p.k_eff > 0) {
        const double wT = (double)sexp(key_to_float(st.tkey) - st.M);
        W += (double)(total_ties - st.ties_needed) * wT;
      }
    }
  }
  st.W = a.w_in ? a.w_in[u] : (float)W;
  if (!(st.flags & (kFlagEmpty | kFlagDense)) && p.m > 0 && p.L - p.k_eff > 0 && st.W > 0.0f)
    st.flags |= kFlagSample;
  if (threadIdx.x == 0) {
    reinterpret_cast<UnitState*>(a.state)[u] = st;
    if (a.norm_out) {
      a.norm_out[2 * u] = st.M;
      a.norm_out[2 * u + 1] = st.W;
    }
  }
}

// ------------------------------------------------------------------ sample
// Per chunk: decide membership of every token (deterministic set, sampled
// tail token, or neither) and write the chunk's segment: deterministic tokens
// in ascending order, then sampled tokens in ascending order.  With emit_rows
// the segment holds cache row numbers (for the fused attention stage) instead
// of positions.
__global__ __launch_bounds__(kNT) void sample_kernel(SelectArgs a) {
  __shared__ float sh[kChunk];
  __shared__ int scan_scr[kNT / 64];

  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / a.Hkv;
  const int h = u - b * a.Hkv;
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  const int c0 = c * kChunk;
  int32_t* cnt = a.sel_cnt + ((size_t)u * a.nchunk + c) * 2;
  if (c0 >= st.L || (st.flags & kFlagEmpty)) {
    if (threadIdx.x == 0) {
      cnt[0] = 0;
      cnt[1] = 0;
    }
    return;
  }
  stage_chunk_scores(a.scores + (size_t)u * a.score_ld, c0, st.L, sh);
  const bool dense = st.flags & kFlagDense;
  const bool notopk = st.flags & kFlagNoTopk;
  const int tb = threadIdx.x * kPer;

  float s[kPer];
  uint32_t validmask = 0u, smask = 0u, tiemask = 0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    s[i] = sh[tb + i];
    const bool valid = c0 + tb + i < st.L;
    validmask |= (uint32_t)valid << i;
    if (valid && !dense && !notopk) {
      const uint32_t key = order_key(s[i]);
      smask |= (uint32_t)(key > st.tkey) << i;
      tiemask |= (uint32_t)(key == st.tkey) << i;
    }
  }
  if (dense) smask = validmask;
  // Tokens on the threshold key join the deterministic set in index order
  // until the quota is met.  Only a chunk that straddles the quota needs the
  // ranks; the branch is uniform over the workgroup.
  if (!dense && !notopk) {
    const size_t ci = (size_t)u * a.nchunk + c;
    const int before = a.ties_before[ci];
    const int here = a.tiecnt[ci];
    if (here > 0) {
      if (before + here <= st.ties_needed) {
        smask |= tiemask;
      } else if (before < st.ties_needed) {
        int tot_unused;
        int rank = before + block_exclusive_scan<kNT>(__popc(tiemask), scan_scr, &tot_unused);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (tiemask & (1u << i)) {
            if (rank < st.ties_needed) smask |= 1u << i;
            ++rank;
          }
        }
      }
    }
  }
  const uint32_t tailmask = validmask & ~smask;
  uint32_t rmask = 0u;
  float logw[kPer];
  if ((st.flags & kFlagSample) && tailmask) {
    const uint64_t seed = a.seed[b];
    const float mf = (float)st.m;
#pragma unroll
    for (int g = 0; g < kPer / 4; ++g) {
      if (((tailmask >> (4 * g)) & 0xfu) == 0u) continue;
      const uint4 wd = philox_block(seed, b, h, (uint32_t)(c0 + tb + 4 * g) >> 2);
      const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        if (!(tailmask & (1u << i))) continue;
        const float w = sexp(s[i] - st.M);
        const float mw = mf * w;
        const float uw = uniform24(words[r]) * st.W;
        if (uw < mw) {
          rmask |= 1u << i;
          logw[i] = -logf(fminf(1.0f, mw / st.W));
        }
      }
    }
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
  const int* btrow = a.block_table + (size_t)b * a.max_blocks;
  int ws = packed & 0xffff, wr = totS + (packed >> 16);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t bit = 1u << i;
    if ((smask | rmask) & bit) {
      const int t = c0 + tb + i;
      int v = t;
      if (a.emit_rows) {
        int blk = btrow[t >> 4];
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        v = (blk * a.Hkv + h) * kBlockTokens + (t & 15);
      }
      if (smask & bit) {
        sidx[ws] = v;
        slw[ws] = 0.0f;
        ++ws;
      } else {
        sidx[wr] = v;
        slw[wr] = logw[i];
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

__global__ void debug_philox_kernel(uint64_t seed, int b, int h, int j0, int n, uint32_t* words) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t j = (uint32_t)(j0 + i);
  const uint4 wd = philox_block(seed, b, h, j >> 2);
  const uint32_t w4[4] = {wd.x, wd.y, wd.z, wd.w};
  words[i] = w4[j & 3u];
}

__global__ void debug_sexp_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = sexp(x[i]);
}

}  // namespace

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

hipError_t launch_sample(const SelectArgs& a, int units, hipStream_t stream) {
  sample_kernel<<<dim3(a.nchunk, units), kNT, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_debug_philox(uint64_t seed, int b, int h, int j0, int n, uint32_t* words,
                               hipStream_t stream) {
  debug_philox_kernel<<<(n + 255) / 256, 256, 0, stream>>>(seed, b, h, j0, n, words);
  return hipGetLastError();
}

hipError_t launch_debug_sexp(const float* x, float* y, int n, hipStream_t stream) {
  debug_sexp_kernel<<<(n + 255) / 256, 256, 0, stream>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace ssa

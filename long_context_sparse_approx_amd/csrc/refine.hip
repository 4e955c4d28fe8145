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
constexpr int kRT = 1024;    // threads of a member's select workgroup
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

// Grid: (chunks, group units) x kRS threads.  LPT lanes per candidate (one
// 16-byte slice of its scored dims each); all the group's members are scored
// from one load of the slice.
template <int LPT>
__global__ __launch_bounds__(kRS) void refine_score_kernel(RefineArgs a) {
  __shared__ float qsh[kRefineQ];
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
  const int rowq = a.G * nd;  // floats per member (the host keeps nmem * rowq <= kRefineQ)
  for (int i = threadIdx.x; i < nmem * rowq; i += kRS) {
    const int mi = i / rowq;
    const int r = i - mi * rowq;
    const int gh = r / nd;
    const int e = r - gh * nd;
    const uint16_t bits =
        a.q[((size_t)(b * a.T + t0 + mi) * a.Hq + h * a.G + gh) * a.d + 2 * a.pair_begin + e];
    qsh[i] = __uint_as_float((uint32_t)bits << 16);
  }
  __syncthreads();
  const int sl = threadIdx.x % LPT;
  const int tk = threadIdx.x / LPT;
  constexpr int TPP = kRS / LPT;  // candidates per pass
  const int32_t* pidx = a.gsel_idx + (size_t)u * a.seg_ld + c0;
  const int* btrow = a.block_table + (size_t)b * a.max_blocks;
  for (int base = 0; base < n_det; base += TPP) {  // uniform trip count
    const int i = base + tk;
    const bool valid = i < n_det;
    const int pos = valid ? min(max(pidx[i], 0), ui.L - 1) : 0;
    int blk = btrow[pos >> 4];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const size_t row = (size_t)(blk * a.Hkv + h) * kBlockTokens + (pos & 15);
    const uint4 kv =
        *reinterpret_cast<const uint4*>(a.k_cache + row * a.key_ld + a.key_off + sl * 8);
    const float kf[8] = {bf16_lo(kv.x), bf16_hi(kv.x), bf16_lo(kv.y), bf16_hi(kv.y),
                         bf16_lo(kv.z), bf16_hi(kv.z), bf16_lo(kv.w), bf16_hi(kv.w)};
    for (int mi = 0; mi < nmem; ++mi) {  // uniform
      float acc = 0.0f;
      for (int gh = 0; gh < a.G; ++gh) {  // uniform
        const float* qs = qsh + mi * rowq + gh * nd + sl * 8;
        float p = qs[0] * kf[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) p = p + qs[e] * kf[e];  // exact products, dim order
#pragma unroll
        for (int x = 1; x < LPT; x <<= 1) p = p + __shfl_xor(p, x);
        acc = gh == 0 ? p : acc + p;
      }
      const float s = acc * a.own_scale;
      if (valid && sl == 0) {
        const int v = (b * a.T + t0 + mi) * a.Hkv + h;
        a.own_key[(size_t)v * a.seg_ld + c0 + i] = order_key(s);
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

// Grid: member units x kRT threads.
__global__ __launch_bounds__(kRT) void refine_select_kernel(RefineArgs a) {
  constexpr int kDig = 4096;
  __shared__ uint32_t hist[kDig];
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
  // Candidate passes: thread t serves chunk (t / tpc) + j * (kRT / tpc) and,
  // inside it, entries (t % tpc) + i * tpc: fixed items, fixed sum orders.
  int tpc = kRT;
  while (tpc > 1 && tpc * nc > kRT) tpc >>= 1;
  const int cstep = kRT / tpc;
  const int csub = threadIdx.x % tpc;
  const size_t cu = (size_t)u * a.nchunk;
  const int32_t* gidx = a.gsel_idx + (size_t)u * a.seg_ld;
  const uint32_t* okey = a.own_key + (size_t)v * a.seg_ld;
  auto each = [&](auto&& f) {
    for (int c = threadIdx.x / tpc; c < nc; c += cstep) {
      const int n = clamp_count(a.gsel_cnt[2 * (cu + c)], kChunk);
      for (int i = csub; i < n; i += tpc) {
        const size_t at = (size_t)c * kChunk + i;
        f(min(max(gidx[at], 0), max(Lg - 1, 0)), at);
      }
    }
  };
  int ncand = 0;
  each([&](int pos, size_t) { ncand += pos < Lt ? 1 : 0; });
  ncand = block_sum_i32<kRT>(ncand, scan);
  const int kt = min(k, ncand);
  int flags = 0;
  if (Lt == 0 || (gs.flags & kFlagEmpty)) flags |= kFlagEmpty;
  else if ((int64_t)kt + m >= (int64_t)Lt) flags |= kFlagDense;
  unsigned long long vstar = 0ull;
  double W = 0.0;
  if (!(flags & (kFlagEmpty | kFlagDense))) {
    if (kt > 0) {
      // Radix select of the kt-th smallest 56-bit word: the inverted own key
      // as digits of 11, 11 and 10 bits, then the position as 12 and 12.
      const int shifts[5] = {45, 34, 24, 12, 0};
      const int widths[5] = {11, 11, 10, 12, 12};
      unsigned long long prefix = 0ull;
      int rank = kt;
      for (int d = 0; d < 5; ++d) {
        const int sh = shifts[d], wd = widths[d];
        for (int i = threadIdx.x; i < kDig; i += kRT) hist[i] = 0u;
        __syncthreads();
        each([&](int pos, size_t at) {
          if (pos >= Lt) return;
          const unsigned long long w = member_word(okey[at], pos);
          if ((w >> (sh + wd)) == prefix)
            atomicAdd(&hist[(w >> sh) & ((1u << wd) - 1u)], 1u);
        });
        __syncthreads();
        int bin, rem;
        find_bin_up(hist, kDig, rank, scan, pair, &bin, &rem);
        prefix = (prefix << wd) | (unsigned long long)bin;
        rank = rem;
      }
      vstar = prefix;
    }
    // W_t: the group's tail sum plus the proxy weight of every candidate the
    // member does not keep (those outside its span included).
    double ws = 0.0;
    const float* srow = a.scores + (size_t)u * a.score_ld;
    each([&](int pos, size_t at) {
      const bool kept = kt > 0 && pos < Lt && member_word(okey[at], pos) <= vstar;
      if (!kept) ws += (double)sexp(srow[pos] - gs.M);
    });
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

// Grid: (chunks, member units) x kRS threads.
__global__ __launch_bounds__(kRS) void refine_emit_kernel(RefineArgs a) {
  __shared__ uint32_t mark[kChunk];
  __shared__ int scan_scr[kRS / 64];
  constexpr int kPerT = kChunk / kRS;
  const int c = blockIdx.x;
  const int v = blockIdx.y;
  int b, t, h, u;
  decode_member(a, v, &b, &t, &h, &u);
  const MemberState ms = reinterpret_cast<const MemberState*>(a.mstate)[v];
  const int c0 = c * kChunk;
  int32_t* cnt = a.msel_cnt + ((size_t)v * a.nchunk + c) * 2;
  if (c0 >= ms.L || (ms.flags & kFlagEmpty)) {
    if (threadIdx.x == 0) {
      cnt[0] = 0;
      cnt[1] = 0;
    }
    return;
  }
  const int nvalid = min(kChunk, ms.L - c0);
  const bool dense = ms.flags & kFlagDense;
  const bool sampling = ms.flags & kFlagSample;
  for (int i = threadIdx.x; i < kChunk; i += kRS)
    mark[i] = (dense && i < nvalid) ? kMarkDet : kMarkNone;
  __syncthreads();
  if (!dense) {
    const size_t ci = (size_t)u * a.nchunk + c;
    const int n_det = clamp_count(a.gsel_cnt[2 * ci], kChunk);
    const int n_smp = clamp_count(a.gsel_cnt[2 * ci + 1], kChunk - n_det);
    const int32_t* gidx = a.gsel_idx + (size_t)u * a.seg_ld + c0;
    const uint32_t* okey = a.own_key + (size_t)v * a.seg_ld + c0;
    const float* srow = a.scores + (size_t)u * a.score_ld;
    const uint64_t seed = a.seed[b];
    const int grp = t / a.g;
    const float mf = (float)ms.m;
    for (int i = threadIdx.x; i < n_det + n_smp; i += kRS) {
      const int pos = gidx[i];
      if ((unsigned)(pos - c0) >= (unsigned)nvalid) continue;  // outside the member's span
      if (i < n_det && !(ms.flags & kFlagNoTopk) && member_word(okey[i], pos) <= ms.vstar) {
        mark[pos - c0] = kMarkDet;
      } else if (sampling) {
        const uint4 wd = philox_block(seed, b, h, (uint32_t)pos >> 2, grp);
        const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
        const float mw = mf * sexp(srow[pos] - ms.M);
        if (uniform24(words[pos & 3]) * ms.W < mw)
          mark[pos - c0] = __float_as_uint(-logf(fminf(1.0f, mw / ms.W)));
      }
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
  const int packed = block_exclusive_scan<kRS>(__popc(smask) | (__popc(rmask) << 16), scan_scr,
                                               &packed_tot);
  const int totS = packed_tot & 0xffff;
  const int totR = packed_tot >> 16;
  int32_t* sidx = a.msel_idx + (size_t)v * a.seg_ld + c0;
  float* slw = a.msel_logw + (size_t)v * a.seg_ld + c0;
  int ws = packed & 0xffff, wr = totS + (packed >> 16);
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const uint32_t bit = 1u << i;
    if ((smask | rmask) & bit) {
      const int pos = c0 + tb + i;
      if (smask & bit) {
        sidx[ws] = pos;
        slw[ws] = 0.0f;
        ++ws;
      } else {
        sidx[wr] = pos;
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

}  // namespace

hipError_t launch_refine(const RefineArgs& a, int group_units, int member_units,
                         hipStream_t stream) {
  const int nmem = a.g < a.T ? a.g : a.T;
  if (nmem * a.G * 2 * a.pair_count > kRefineQ) return hipErrorInvalidValue;
  const dim3 sg(a.nchunk, group_units);
  switch (a.pair_count / 4) {  // lanes per candidate: 2 * pair_count / 8
    case 1: refine_score_kernel<1><<<sg, kRS, 0, stream>>>(a); break;
    case 2: refine_score_kernel<2><<<sg, kRS, 0, stream>>>(a); break;
    case 4: refine_score_kernel<4><<<sg, kRS, 0, stream>>>(a); break;
    case 8: refine_score_kernel<8><<<sg, kRS, 0, stream>>>(a); break;
    case 16: refine_score_kernel<16><<<sg, kRS, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  refine_select_kernel<<<member_units, kRT, 0, stream>>>(a);
  refine_emit_kernel<<<dim3(a.nchunk, member_units), kRS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ssa
